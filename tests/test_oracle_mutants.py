"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The mutants are textual edits of ``oracle/oracle.c`` compiled into temporary
libraries on the CPU; the real oracle is never modified.  If an edit's target
text is no longer found, the test fails loudly so the list stays in step with
the source.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "drop_skip_term": ("double pre = s + dval * xv;", "double pre = s;"),
    "wrong_sign_in_exp": ("*abar = exp(u);", "*abar = exp(-u);"),
    "euler_instead_of_zoh": ("*bbar_coef = (a != 0.0) ? expm1(u) / a : delta;",
                             "*bbar_coef = delta;"),
    "zero_A_limit_wrong": ("*bbar_coef = (a != 0.0) ? expm1(u) / a : delta;",
                           "*bbar_coef = (a != 0.0) ? expm1(u) / a : 0.0;"),
    "C_used_for_B": ("bcoef * B[bc + n] * xv", "bcoef * C[bc + n] * xv"),
    "state_index_reversed": ("a_row[n * a_step]", "a_row[(dstate - 1 - n) * a_step]"),
    "euler_drops_delta": ("*bbar_coef = delta;\n}", "*bbar_coef = 1.0;\n}"),
    "euler_uses_the_hold": ("*bbar_coef = delta;\n}", "*bbar_coef = expm1(delta * a) / a;\n}"),
    "euler_linear_decay": ("*abar = exp(delta * a);", "*abar = 1.0 + delta * a;"),
    "per_channel_A_of_channel_0": ("a_per_channel ? A + d : A + d * dstate",
                                   "a_per_channel ? A : A + d * dstate"),
    "per_channel_A_stepped": ("a_per_channel ? 0 : 1", "1"),
    "bwd_coef_derivative_dropped": ("g->dcoef_dd = g->abar;", "g->dcoef_dd = 1.0;"),
    "bwd_dcoef_da_sign": ("g->dcoef_da = (delta * g->abar - g->coef) / a;",
                          "g->dcoef_da = (g->coef - delta * g->abar) / a;"),
    "bwd_zero_A_limit_dropped": ("g->dcoef_da = 0.5 * delta * delta;", "g->dcoef_da = 0.0;"),
    "bwd_adjoint_not_decayed": ("e[n] = g.abar * dh;", "e[n] = dh;"),
    "bwd_dC_from_previous_state": ("dC_acc[bc + n] += dp * h_t[n];",
                                   "dC_acc[bc + n] += dp * h_prev[n];"),
    "bwd_dB_without_coef": ("dB_acc[bc + n] += dh * g.coef * xv;", "dB_acc[bc + n] += dh * xv;"),
    "bwd_gate_derivative_is_sigmoid": ("return sg * (1.0 + v * (1.0 - sg));", "return sg;"),
    "bwd_dh_last_ignored": ("e[n] = dh_last_row ? dh_last_row[n] : 0.0;", "e[n] = 0.0;"),
    "bwd_skip_in_dx_dropped": ("double dxv = dp * dval, ddv = 0.0;",
                               "double dxv = 0.0, ddv = 0.0;"),
    "bwd_ddelta_uses_new_state": ("ddv += dh * (g.dabar_dd * h_prev[n]",
                                  "ddv += dh * (g.dabar_dd * h_t[n]"),
    "no_decay": ("h[n] = abar * h[n] + bcoef", "h[n] = h[n] + bcoef"),
    "previous_token_B_C": ("int64_t bc = (b * seqlen + t) * dstate;",
                           "int64_t bc = (b * seqlen + (t > 0 ? t - 1 : 0)) * dstate;"),
    "h0_ignored": ("h[n] = h0 ? h0[ch * dstate + n] : 0.0;", "h[n] = 0.0;"),
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "gate_without_silu": ("pre * silu(z[io])", "pre * z[io]"),
    "readout_before_update": (
        "        /* state update first: h_t = Abar_t h_{t-1} + Bbar_t x_t */",
        "        double s0 = 0.0;\n"
        "        for (int64_t n = 0; n < dstate; ++n) s0 += C[bc + n] * h[n];"),
    "conv_taps_reversed": ("acc += w[d * d_conv + k] * x_raw",
                           "acc += w[d * d_conv + (d_conv - 1 - k)] * x_raw"),
    "conv_one_step_late": ("int64_t ts = t - (d_conv - 1) + k;",
                           "int64_t ts = t - d_conv + k;"),
    "conv_bias_dropped": ("double acc = bias ? bias[d] : 0.0;", "double acc = 0.0;"),
    "softplus_sign": ("log1p(exp(-fabs(v)))", "log1p(exp(fabs(v)))"),
    "softplus_bias_dropped": ("softplus(delta_raw[i * dim + d] + (bias ? bias[d] : 0.0))",
                              "softplus(delta_raw[i * dim + d])"),
    "half_state_read": ("for (int64_t n = 0; n < dstate; ++n) s += C[bc + n] * h[n];",
                        "for (int64_t n = 0; n < dstate / 2; ++n) s += C[bc + n] * h[n];"),
}


def _fixup(name, src):
    # the readout-before-update mutant also needs the readout to use s0
    if name == "readout_before_update":
        src = src.replace("double pre = s + dval * xv;", "double pre = s0 + dval * xv;")
    return src


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle._SRC) as f:
        src = f.read()
    assert old in src, f"mutation target for {name!r} not found in oracle.c"
    src = _fixup(name, src.replace(old, new, 1))
    path = tmp_path / "mutant.c"
    path.write_text(src)
    so = oracle.build(str(path), str(tmp_path / "libmutant.so"))
    lib = oracle.load_library(so)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name!r} passed every pin"
