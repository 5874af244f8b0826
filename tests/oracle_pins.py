"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load_library``)
and raises AssertionError when the oracle disagrees with what the pages or
mathematics fix.  ``test_oracle_pins.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on copies of the oracle with a planted
mistake, each of which must be caught by at least one pin.

What pins what (pages cited by title and section):

* ZOH discretisation: integrating the continuous system h' = A h + B x with x
  held over the step (RK4, 10^4 substeps) must land on Abar h0 + Bbar x
  (paperlens tutorial, eq.(1)/(2) and the zero-order-hold prose; ultralytics
  glossary, section on how SSMs work).
* Recurrence and readout: with delta, B, C constant the scan must equal the
  convolution with kernel K_k = C . (Abar^k * Bbar), re-running the glossary's
  worked example (L=64, N=16, delta=0.1) and random variants (ultralytics
  glossary worked example; paperlens tutorial, section "S4: 再帰は畳み込みでもある").
* delta -> 0 leaves the state unchanged; large delta overwrites it with the
  current input (paperlens tutorial, prose under eq.(2) and the selection
  section).
* Brute force: explicit unrolled products/sums on tiny inputs.
* Closed form of one step with the D term and the SiLU gate (ihouse article,
  output equation; agenticai-flow guide, block diagram).
* Linearity in (x, h0) without the gate, and associativity of chunking
  (paperlens tutorial, section on the parallel scan).
* L decode steps equal one scan (paperlens tutorial, S4 section: recurrent and
  convolutional faces give the same outputs).
* Backward: every gradient (x, delta, A, B, C, D, z, h0) against central
  differences of the forward oracle, for both rules, A per channel and A = 0;
  and Euler's theorem on homogeneous functions for x, B and C (y is linear
  in each when there is no gate, skip or initial state).
* Variants: the Euler rule Bbar = delta*B against brute force, its one-step
  closed form, and its second-order agreement with the hold for small delta;
  A given per channel against brute force with A broadcast over the states,
  and the single decay rate it implies (paperlens tutorial, selection
  pseudo-code; ihouse article, Mamba-2 section); a step and decay shared by
  a head of channels against the masked-matrix form of the same scan
  (ihouse article, section on Mamba's evolution), and the gradients of the
  head-shared dt and A against central differences.
* Prologue of the fused scan (paperlens tutorial, sections "現場ではこう使う"
  and "Mamba: 状態を「選択的」にする"): the causal depthwise convolution equals
  numpy's convolve of each channel with its reversed taps, and cannot see the
  future; softplus satisfies softplus(0) = ln 2 and softplus(v) - softplus(-v) = v
  and has the right asymptotes; the bias is added before the softplus.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _rand_problem(rng, b, L, d, n, with_d=True, with_z=True, with_h0=True,
                  dmin=0.001, dmax=0.5):
    x = rng.standard_normal((b, L, d))
    delta = rng.uniform(dmin, dmax, (b, L, d))
    A = -rng.uniform(0.5, 1.5, (d, n))
    B = rng.standard_normal((b, L, n))
    C = rng.standard_normal((b, L, n))
    D = rng.standard_normal(d) if with_d else None
    z = rng.standard_normal((b, L, d)) if with_z else None
    h0 = rng.standard_normal((b, d, n)) if with_h0 else None
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=D, z=z, h0=h0)


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


# --------------------------------------------------------------------------
# ZOH against the ODE it discretises
# --------------------------------------------------------------------------
def _rk4_step_diag(a, bx, h, dt):
    k1 = a * h + bx
    k2 = a * (h + 0.5 * dt * k1) + bx
    k3 = a * (h + 0.5 * dt * k2) + bx
    k4 = a * (h + dt * k3) + bx
    return h + dt / 6.0 * (k1 + 2 * k2 + 2 * k3 + k4)


def _integrate(a, bx, h0, delta, steps=10_000):
    """h' = a h + bx over [0, delta] from h0, classic RK4 (vectorised over n)."""
    h = np.array(h0, dtype=np.float64)
    dt = delta / steps
    for _ in range(steps):
        h = _rk4_step_diag(a, bx, h, dt)
    return h


def pin_zoh_matches_ode(lib):
    rng = _rng(11)
    n = 8
    for delta in (1e-3, 0.05, 0.3, 1.7):
        A = np.concatenate([-rng.uniform(0.5, 1.5, n - 2), [0.7, -3e-4]])
        B = rng.standard_normal(n)
        x = float(rng.standard_normal())
        h0 = rng.standard_normal(n)
        _, h_last = oracle.scan(np.full((1, 1, 1), x), np.full((1, 1, 1), delta),
                                A[None, :], B[None, None, :], np.zeros((1, 1, n)),
                                h0=h0[None, None, :], lib=lib)
        ref = _integrate(A, B * x, h0, delta)
        err = np.max(np.abs(h_last[0, 0] - ref) / (1.0 + np.abs(ref)))
        assert err < 1e-12, f"ZOH vs ODE (delta={delta}): {err}"


# --------------------------------------------------------------------------
# Recurrence against the convolution form (constant delta, B, C)
# --------------------------------------------------------------------------
def _conv_form(A, B, C, delta, x):
    """Output of the time-invariant system as a causal convolution: the
    impulse response at lag k is K_k = sum_n C_n Abar_n^k Bbar_n, and y is
    the first L terms of the full convolution of x with K."""
    L = len(x)
    gain = C * B * np.expm1(delta * A) / A                   # C_n Bbar_n
    decay = np.exp(delta * A)                                 # Abar_n
    lags = np.ones((L, len(A)))                               # Abar_n^k, k = 0 .. L-1
    lags[1:] = decay
    lags = np.cumprod(lags, axis=0)
    return np.convolve(x, lags @ gain)[:L]


def _scan_const(lib, A, B, C, delta, x):
    L, n = len(x), len(A)
    y, _ = oracle.scan(x.reshape(1, L, 1), np.full((1, L, 1), delta), A[None, :],
                       np.broadcast_to(B, (1, L, n)), np.broadcast_to(C, (1, L, n)),
                       lib=lib)
    return y[0, :, 0]


def pin_worked_example_recurrence_equals_convolution(lib):
    with open(os.path.join(GOLDEN, "worked_example_recurrence_vs_convolution.json")) as f:
        g = json.load(f)
    import torch  # the example draws its inputs with torch's seeded CPU RNG

    torch.manual_seed(g["torch_seed"])
    L, N = g["L"], g["N"]
    x = torch.randn(L).double().numpy()
    A = (-(torch.rand(N) + 0.5)).double().numpy()
    B = torch.randn(N).double().numpy()
    C = torch.randn(N).double().numpy()
    delta = g["delta"]
    y_rec = _scan_const(lib, A, B, C, delta, x)
    y_conv = _conv_form(A, B, C, delta, x)
    # the page's own check (atol 1e-5) reports True ...
    assert bool(np.allclose(y_rec, y_conv, atol=g["atol"], rtol=0)) == g["expected"]
    # ... and in fp64 the two forms agree to rounding
    assert _rel(y_rec, y_conv) < 1e-12


def pin_random_recurrence_equals_convolution(lib):
    rng = _rng(12)
    for L, n, delta in ((40, 4, 0.02), (97, 16, 0.3), (33, 7, 1.3)):
        A = -rng.uniform(0.05, 2.0, n)
        B, C, x = rng.standard_normal(n), rng.standard_normal(n), rng.standard_normal(L)
        assert _rel(_scan_const(lib, A, B, C, delta, x), _conv_form(A, B, C, delta, x)) < 1e-12


# --------------------------------------------------------------------------
# delta limits
# --------------------------------------------------------------------------
def pin_delta_zero_keeps_state(lib):
    rng = _rng(13)
    p = _rand_problem(rng, 2, 9, 3, 5)
    p["delta"] = np.zeros_like(p["delta"])
    y, h_last = oracle.scan(lib=lib, **p)
    assert np.array_equal(h_last, p["h0"]), "delta=0 must leave the state bit-for-bit"
    # y_t = (C_t . h0 + D x_t) * SiLU(z_t)
    ch = np.einsum("bln,bdn->bld", p["C"], p["h0"])
    ref = (ch + p["D"][None, None, :] * p["x"]) * _silu(p["z"])
    assert _rel(y, ref) < 1e-14


def pin_large_delta_overwrites_state(lib):
    rng = _rng(14)
    p = _rand_problem(rng, 1, 6, 2, 4, with_z=False, with_d=False)
    p["delta"] = np.full_like(p["delta"], 60.0)
    p["A"] = -rng.uniform(0.5, 1.5, p["A"].shape)
    y, h_last = oracle.scan(lib=lib, **p)
    # state forgets everything but the last token: h = -B x / A
    ref_h = -p["B"][0, -1][None, :] * p["x"][0, -1][:, None] / p["A"]
    assert _rel(h_last[0], ref_h) < 1e-12
    ref_y = np.einsum("ln,ldn->ld", p["C"][0],
                      -p["B"][0][:, None, :] * p["x"][0][:, :, None] / p["A"][None])
    assert _rel(y[0], ref_y) < 1e-12


# --------------------------------------------------------------------------
# brute force, closed form, linearity, chunking, decode
# --------------------------------------------------------------------------
def _brute_force(p, euler=False):
    """Unrolled products and sums.  A may be [d] (one value per channel, used
    for each of its states); euler=True uses Bbar = delta * B."""
    x, delta, A, B, C, D, z, h0 = (p[k] for k in ("x", "delta", "A", "B", "C", "D", "z", "h0"))
    b, L, d = x.shape
    n = B.shape[2]
    if A.ndim == 1:
        A = np.repeat(A[:, None], n, axis=1)
    y = np.zeros_like(x)
    for bi in range(b):
        for di in range(d):
            a = [np.exp(delta[bi, s, di] * A[di]) for s in range(L)]          # Abar_s
            if euler:
                u = [delta[bi, s, di] * B[bi, s] * x[bi, s, di] for s in range(L)]
            else:
                u = [(a[s] - 1.0) / A[di] * B[bi, s] * x[bi, s, di] for s in range(L)]
            for t in range(L):
                h = np.prod(a[: t + 1], axis=0) * (h0[bi, di] if h0 is not None else 0.0)
                for s in range(t + 1):
                    decay = np.prod(a[s + 1: t + 1], axis=0) if s < t else np.ones(n)
                    h = h + decay * u[s]
                pre = C[bi, t] @ h + (D[di] if D is not None else 0.0) * x[bi, t, di]
                y[bi, t, di] = pre * _silu(z[bi, t, di]) if z is not None else pre
    return y


def pin_brute_force_tiny(lib):
    rng = _rng(15)
    for (b, L, d, n) in ((1, 1, 1, 1), (2, 7, 3, 4), (1, 16, 4, 2), (2, 5, 2, 3)):
        for flags in ((True, True, True), (False, False, False), (True, False, True)):
            p = _rand_problem(rng, b, L, d, n, *flags)
            y, _ = oracle.scan(lib=lib, **p)
            assert _rel(y, _brute_force(p)) < 1e-12, (b, L, d, n, flags)


def pin_single_step_closed_form(lib):
    rng = _rng(16)
    for _ in range(5):
        delta, a = rng.uniform(0.01, 2.0), -rng.uniform(0.1, 3.0)
        x, h0, Bv, Cv, Dv, zv = rng.standard_normal(6)
        y, h = oracle.scan(np.full((1, 1, 1), x), np.full((1, 1, 1), delta),
                           np.full((1, 1), a), np.full((1, 1, 1), Bv),
                           np.full((1, 1, 1), Cv), np.full(1, Dv),
                           np.full((1, 1, 1), zv), np.full((1, 1, 1), h0), lib=lib)
        abar = np.exp(delta * a)
        hn = abar * h0 + (abar - 1.0) / a * Bv * x
        ref = (Cv * hn + Dv * x) * zv / (1.0 + np.exp(-zv))
        assert abs(y[0, 0, 0] - ref) <= 1e-14 * (1 + abs(ref))
        assert abs(h[0, 0, 0] - hn) <= 1e-14 * (1 + abs(hn))


def pin_linearity(lib):
    rng = _rng(17)
    p1 = _rand_problem(rng, 2, 20, 3, 6, with_z=False)
    p2 = dict(p1, x=rng.standard_normal(p1["x"].shape), h0=rng.standard_normal(p1["h0"].shape))
    al, be = 0.7, -1.9
    p3 = dict(p1, x=al * p1["x"] + be * p2["x"], h0=al * p1["h0"] + be * p2["h0"])
    (y1, h1), (y2, h2), (y3, h3) = (oracle.scan(lib=lib, **p) for p in (p1, p2, p3))
    assert _rel(y3, al * y1 + be * y2) < 1e-12
    assert _rel(h3, al * h1 + be * h2) < 1e-12


# --------------------------------------------------------------------------
# variants: Euler rule Bbar = delta*B, and A as one value per channel
# --------------------------------------------------------------------------
def pin_euler_brute_force_tiny(lib):
    rng = _rng(23)
    for (b, L, d, n) in ((1, 1, 1, 1), (2, 7, 3, 4), (1, 12, 2, 5)):
        p = _rand_problem(rng, b, L, d, n)
        y, _ = oracle.scan(lib=lib, discretization="euler", **p)
        assert _rel(y, _brute_force(p, euler=True)) < 1e-12, (b, L, d, n)


def pin_euler_single_step_closed_form(lib):
    rng = _rng(24)
    for _ in range(5):
        delta, a = rng.uniform(0.01, 2.0), -rng.uniform(0.1, 3.0)
        x, h0, Bv = rng.standard_normal(3)
        _, h = oracle.scan(np.full((1, 1, 1), x), np.full((1, 1, 1), delta),
                           np.full((1, 1), a), np.full((1, 1, 1), Bv), np.zeros((1, 1, 1)),
                           h0=np.full((1, 1, 1), h0), lib=lib, discretization="euler")
        hn = np.exp(delta * a) * h0 + delta * Bv * x
        assert abs(h[0, 0, 0] - hn) <= 1e-14 * (1 + abs(hn))


def pin_euler_agrees_with_zoh_to_second_order(lib):
    """(exp(delta a) - 1)/a = delta + a delta^2 / 2 + O(delta^3): one step
    from h0 = 0 differs between the two rules by a delta^2 B x / 2."""
    rng = _rng(25)
    a = -rng.uniform(0.5, 2.0, 4)
    Bv, x = rng.standard_normal(4), 0.8
    for delta in (1e-2, 1e-3):
        args = (np.full((1, 1, 1), x), np.full((1, 1, 1), delta), a[None, :],
                Bv[None, None, :], np.zeros((1, 1, 4)))
        _, hz = oracle.scan(*args, lib=lib)
        _, he = oracle.scan(*args, lib=lib, discretization="euler")
        lead = a * delta ** 2 / 2 * Bv * x
        assert np.all(np.abs((hz - he)[0, 0] - lead) <= 2 * np.abs(a) ** 2 * delta ** 3 * abs(x)
                      * np.abs(Bv)), delta


def pin_per_channel_A_brute_force(lib):
    rng = _rng(26)
    for euler in (False, True):
        for (b, L, d, n) in ((1, 4, 3, 5), (2, 9, 4, 3)):
            p = _rand_problem(rng, b, L, d, n)
            p["A"] = -rng.uniform(0.2, 2.0, d)
            y, h = oracle.scan(lib=lib, discretization="euler" if euler else "zoh", **p)
            assert _rel(y, _brute_force(p, euler=euler)) < 1e-12, (euler, b, L, d, n)
            # the state decays at the channel's single rate
            if L and not euler:
                q = dict(p, x=np.zeros_like(p["x"]))
                _, hq = oracle.scan(lib=lib, **q)
                rate = np.exp(p["A"][None, :] * p["delta"].sum(axis=1))
                assert _rel(hq, p["h0"] * rate[:, :, None]) < 1e-12


def _masked_matrix_form(x, dt, A, B, C, D, z, h0, P, euler):
    """The scan with a head-shared step written as one masked matrix product per
    (batch row, head): y = (Lmask * (C B^T) * coef) X + exp(cum) * (C h0^T), with
    Lmask[t, s] = exp(A * sum(dt over s < r <= t)) for s <= t, 0 above the
    diagonal (ihouse article, section on Mamba's evolution: the SSM
    computation as a masked matrix multiplication).  Also returns the final
    state.  Written independently of the recurrence."""
    b, L, dim = x.shape
    H, n = dt.shape[2], B.shape[2]
    y = np.zeros_like(x)
    hl = np.zeros((b, dim, n))
    for bi in range(b):
        for h in range(H):
            a = dt[bi, :, h] * A[h]
            cum = np.cumsum(a)
            if euler or A[h] == 0.0:
                coef = dt[bi, :, h]
            else:
                coef = np.expm1(a) / A[h]
            diff = cum[:, None] - cum[None, :]
            lower = np.tril(np.ones((L, L), dtype=bool))
            lmask = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
            M = (C[bi] @ B[bi].T) * lmask * coef[None, :]
            cols = slice(h * P, (h + 1) * P)
            X = x[bi, :, cols]
            Y = M @ X
            w = np.exp(cum[-1] - cum) * coef if L else coef
            S = (X * w[:, None]).T @ B[bi]                                  # [P, n]
            if h0 is not None:
                Y = Y + np.exp(cum)[:, None] * (C[bi] @ h0[bi, cols, :].T)
                S = S + (np.exp(cum[-1]) if L else 1.0) * h0[bi, cols, :]
            pre = Y + (D[cols][None, :] * X if D is not None else 0.0)
            y[bi, :, cols] = pre * _silu(z[bi, :, cols]) if z is not None else pre
            hl[bi, cols, :] = S
    return y, hl


def pin_head_shared_step_equals_masked_matrix_form(lib):
    rng = _rng(27)
    for euler in (False, True):
        for (b, L, H, P, n) in ((1, 1, 1, 1, 1), (2, 9, 2, 3, 4), (1, 20, 3, 2, 5)):
            dim = H * P
            p = _rand_problem(rng, b, L, dim, n)
            dt = rng.uniform(0.001, 0.5, (b, L, H))
            A = -rng.uniform(0.2, 2.0, H)
            if H > 1:
                A[1] = 0.0                       # the delta*B limit of the hold
            y, hl = oracle.scan_heads(p["x"], dt, A, p["B"], p["C"], p["D"], p["z"], p["h0"],
                                      headdim=P, lib=lib,
                                      discretization="euler" if euler else "zoh")
            yr, hr = _masked_matrix_form(p["x"], dt, A, p["B"], p["C"], p["D"], p["z"], p["h0"],
                                         P, euler)
            assert _rel(y, yr) < 1e-12, (euler, b, L, H, P, n)
            assert _rel(hl, hr) < 1e-12, (euler, b, L, H, P, n)


def pin_head_shared_backward_matches_finite_differences(lib):
    """ddt and dA of the per-head scan against central differences of
    ``scan_heads`` (the other gradients are those of the per-channel backward,
    pinned below)."""
    rng = _rng(28)
    for euler in (False, True):
        b, L, H, P, n = 2, 7, 2, 3, 4
        p = _rand_problem(rng, b, L, H * P, n)
        dt = rng.uniform(0.05, 0.5, (b, L, H))
        A = -rng.uniform(0.3, 1.5, H)
        dy = rng.standard_normal(p["x"].shape)
        dhl = rng.standard_normal(p["h0"].shape)
        disc = "euler" if euler else "zoh"
        g = oracle.scan_heads_bwd(p["x"], dt, A, p["B"], p["C"], p["D"], p["z"], p["h0"],
                                  dy=dy, dh_last=dhl, headdim=P, lib=lib, discretization=disc)

        def loss(dt_, A_):
            y, h = oracle.scan_heads(p["x"], dt_, A_, p["B"], p["C"], p["D"], p["z"], p["h0"],
                                     headdim=P, lib=lib, discretization=disc)
            return float(np.sum(dy * y) + np.sum(dhl * h))

        eps = 1e-6
        for idx in [(0, 0, 0), (1, 3, 1), (0, 6, 1), (1, 0, 0)]:
            dp, dm = dt.copy(), dt.copy()
            dp[idx] += eps
            dm[idx] -= eps
            fd = (loss(dp, A) - loss(dm, A)) / (2 * eps)
            assert abs(g["ddt"][idx] - fd) <= 1e-6 * (1 + abs(fd)), (disc, idx, g["ddt"][idx], fd)
        for h in range(H):
            ap, am = A.copy(), A.copy()
            ap[h] += eps
            am[h] -= eps
            fd = (loss(dt, ap) - loss(dt, am)) / (2 * eps)
            assert abs(g["dA"][h] - fd) <= 1e-6 * (1 + abs(fd)), (disc, h, g["dA"][h], fd)


# --------------------------------------------------------------------------
# backward: every gradient against central differences of the forward oracle
# --------------------------------------------------------------------------
def _loss(lib, p, dy, dhl, disc):
    y, h = oracle.scan(lib=lib, discretization=disc, **p)
    return float(np.sum(dy * y) + (np.sum(dhl * h) if dhl is not None else 0.0))


def _check_grads_fd(lib, p, dy, dhl, disc, rng, per_tensor=12):
    g = oracle.scan_bwd(lib=lib, dy=dy, dh_last=dhl, discretization=disc, **p)
    names = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "z": "dz", "h0": "dh0"}
    for k, gk in names.items():
        if p.get(k) is None:
            continue
        v = p[k]
        flat = rng.choice(v.size, size=min(per_tensor, v.size), replace=False)
        for i in flat:
            idx = np.unravel_index(i, v.shape)
            eps = 1e-6 * max(1.0, abs(v[idx]))
            orig = v[idx]
            v[idx] = orig + eps
            lp = _loss(lib, p, dy, dhl, disc)
            v[idx] = orig - eps
            lm = _loss(lib, p, dy, dhl, disc)
            v[idx] = orig
            fd = (lp - lm) / (2 * eps)
            an = g[gk][idx]
            assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (disc, k, idx, fd, an)


def pin_backward_matches_finite_differences(lib):
    rng = _rng(27)
    for disc in ("zoh", "euler"):
        for (b, L, d, n, flags) in ((2, 6, 3, 4, (True, True, True)),
                                    (1, 9, 2, 3, (False, False, False))):
            p = _rand_problem(rng, b, L, d, n, *flags)
            dy = rng.standard_normal(p["x"].shape)
            dhl = rng.standard_normal((b, d, n)) if flags[2] else None
            _check_grads_fd(lib, p, dy, dhl, disc, rng)


def pin_backward_variants_and_zero_A(lib):
    """A per channel, and A entries of exactly 0 (the limit of the hold)."""
    rng = _rng(28)
    p = _rand_problem(rng, 2, 7, 3, 4)
    p["A"][1, 2] = 0.0
    p["A"][2, :] = 0.0
    dy = rng.standard_normal(p["x"].shape)
    _check_grads_fd(lib, p, dy, rng.standard_normal((2, 3, 4)), "zoh", rng, per_tensor=20)
    for disc in ("zoh", "euler"):
        q = _rand_problem(rng, 2, 5, 3, 4)
        q["A"] = -rng.uniform(0.2, 2.0, 3)
        _check_grads_fd(lib, q, rng.standard_normal(q["x"].shape),
                        rng.standard_normal((2, 3, 4)), disc, rng)


def pin_backward_gradient_of_a_linear_readout(lib):
    """With no gate, D = 0 and h0 = 0, y is linear in x: sum(dy * y) equals
    sum(dx * x) exactly (Euler's theorem for homogeneous functions)."""
    rng = _rng(29)
    p = _rand_problem(rng, 2, 11, 3, 5, with_d=False, with_z=False, with_h0=False)
    dy = rng.standard_normal(p["x"].shape)
    y, _ = oracle.scan(lib=lib, **p)
    g = oracle.scan_bwd(lib=lib, dy=dy, **p)
    assert abs(np.sum(dy * y) - np.sum(g["dx"] * p["x"])) <= 1e-12 * np.sum(np.abs(dy * y))
    # y is also linear in B and in C separately
    assert abs(np.sum(dy * y) - np.sum(g["dB"] * p["B"])) <= 1e-12 * np.sum(np.abs(dy * y))
    assert abs(np.sum(dy * y) - np.sum(g["dC"] * p["C"])) <= 1e-12 * np.sum(np.abs(dy * y))


def _slice_t(p, lo, hi):
    q = dict(p)
    for k in ("x", "delta", "B", "C", "z"):
        if q[k] is not None:
            q[k] = np.ascontiguousarray(q[k][:, lo:hi])
    return q


def pin_chunk_split(lib):
    rng = _rng(18)
    p = _rand_problem(rng, 2, 50, 3, 5)
    y, h = oracle.scan(lib=lib, **p)
    for cut in (1, 17, 49):
        ya, ha = oracle.scan(lib=lib, **_slice_t(p, 0, cut))
        yb, hb = oracle.scan(lib=lib, **dict(_slice_t(p, cut, 50), h0=ha))
        assert _rel(np.concatenate([ya, yb], axis=1), y) < 1e-12
        assert _rel(hb, h) < 1e-12


def pin_decode_equals_scan(lib):
    rng = _rng(19)
    p = _rand_problem(rng, 2, 12, 4, 6)
    y, h_last = oracle.scan(lib=lib, **p)
    h = np.ascontiguousarray(p["h0"].copy())
    for t in range(12):
        yt = oracle.decode_step(h, p["x"][:, t], p["delta"][:, t], p["A"], p["B"][:, t],
                                p["C"][:, t], p["D"], p["z"][:, t], lib=lib)
        assert _rel(yt, y[:, t]) < 1e-12
    assert _rel(h, h_last) < 1e-12


def pin_stability_bound(lib):
    rng = _rng(20)
    p = _rand_problem(rng, 1, 200, 2, 8, with_z=False, with_d=False)
    _, h = oracle.scan(lib=lib, **p)
    bound = np.abs(p["h0"][0]).copy()
    for s in range(200):
        abar = np.exp(p["delta"][0, s][:, None] * p["A"])
        bound += np.abs((abar - 1) / p["A"] * p["B"][0, s][None, :] * p["x"][0, s][:, None])
    assert np.all(np.abs(h[0]) <= bound * (1 + 1e-12))


def pin_zero_A_is_the_limit(lib):
    rng = _rng(21)
    p = _rand_problem(rng, 1, 30, 2, 3)
    p["A"][:, 1] = 0.0
    y0, h0 = oracle.scan(lib=lib, **p)
    for eps in (1e-9, -1e-9):
        q = dict(p, A=p["A"].copy())
        q["A"][:, 1] = eps
        y1, h1 = oracle.scan(lib=lib, **q)
        assert _rel(y0, y1) < 1e-7 and _rel(h0, h1) < 1e-7


def pin_empty_sequence(lib):
    rng = _rng(22)
    p = _rand_problem(rng, 2, 0, 3, 4)
    y, h = oracle.scan(lib=lib, **p)
    assert y.shape == (2, 0, 3) and np.array_equal(h, p["h0"])
    q = dict(p, h0=None)
    _, h = oracle.scan(lib=lib, **q)
    assert np.all(h == 0.0)


# --------------------------------------------------------------------------
# Prologue: causal depthwise conv1d and softplus of delta
# --------------------------------------------------------------------------

def pin_conv1d_matches_numpy_convolve(lib):
    rng = _rng(31)
    b, L, d = 2, 37, 5
    for K in (1, 2, 4):
        x = rng.standard_normal((b, L, d))
        w = rng.uniform(-1, 1, (d, K))
        bias = rng.standard_normal(d)
        out = oracle.conv1d(x, w, bias, silu=False, lib=lib)
        ref = np.empty_like(x)
        for bb in range(b):
            for dd in range(d):
                ref[bb, :, dd] = np.convolve(x[bb, :, dd], w[dd, ::-1])[:L] + bias[dd]
        assert _rel(out, ref) < 1e-14, K
        out0 = oracle.conv1d(x, w, None, silu=False, lib=lib)
        assert _rel(out0 + bias, ref) < 1e-14


def pin_conv1d_is_causal(lib):
    rng = _rng(32)
    x = rng.standard_normal((1, 20, 3))
    w = rng.uniform(0.5, 1.0, (3, 4))  # taps bounded away from zero
    y0 = oracle.conv1d(x, w, None, silu=True, lib=lib)
    x2 = x.copy()
    x2[0, 9, :] += 1.0
    y1 = oracle.conv1d(x2, w, None, silu=True, lib=lib)
    assert np.array_equal(y0[0, :9], y1[0, :9])
    assert np.all(y0[0, 9:13] != y1[0, 9:13])
    assert np.array_equal(y0[0, 13:], y1[0, 13:])


def pin_conv1d_silu_is_applied_after_the_bias(lib):
    rng = _rng(33)
    x = rng.standard_normal((1, 16, 4))
    w = rng.uniform(-1, 1, (4, 3))
    bias = rng.standard_normal(4)
    lin = oracle.conv1d(x, w, bias, silu=False, lib=lib)
    act = oracle.conv1d(x, w, bias, silu=True, lib=lib)
    # SiLU(v) - SiLU(-v) = v, whatever the form of the sigmoid
    neg = oracle.conv1d(-x, w, -bias, silu=True, lib=lib)
    assert _rel(act - neg, lin) < 1e-13
    assert _rel(act, _silu(lin)) < 1e-13


def pin_softplus_values(lib):
    import math
    sp = lib.oracle_softplus
    assert abs(sp(0.0) - math.log(2.0)) < 1e-16
    rng = _rng(34)
    for v in rng.uniform(-30, 30, 200):
        a, b = sp(v), sp(-v)
        assert a > 0.0 and b > 0.0
        assert abs((a - b) - v) <= 1e-14 * max(1.0, abs(v))
    assert abs(sp(60.0) - 60.0) < 1e-13  # softplus(v) = v + log1p(exp(-v))
    assert abs(sp(-40.0) / math.exp(-40.0) - 1.0) < 1e-15


def pin_delta_softplus_adds_the_bias_first(lib):
    rng = _rng(35)
    raw = 0.5 * rng.standard_normal((2, 9, 6))
    bias = rng.uniform(-6, -1, 6)
    dp = oracle.delta_softplus(raw, bias, lib=lib)
    dn = oracle.delta_softplus(-raw, -bias, lib=lib)
    assert _rel(dp - dn, raw + bias) < 1e-13
    assert np.all(dp > 0)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
