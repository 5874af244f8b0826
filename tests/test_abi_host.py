"""C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments before touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

import selective_state_space_44_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation


@pytest.fixture(scope="module")
def lib():
    return ssm.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert {"ssm_scan_fwd", "ssm_decode_step"} <= set(names)
    assert set(names) == set(ssm.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.ssm_abi_version() == 3
    for code in range(5):
        assert lib.ssm_status_str(code).startswith(b"SSM_")
    assert b"UNKNOWN" in lib.ssm_status_str(99)


def _scan(lib, batch=2, L=8, dim=64, N=16, io=1, x=FAKE, delta=FAKE, A=FAKE, B=FAKE,
          C=FAKE, D=None, z=None, h0=None, y=ctypes.c_void_p(0x2000), h_last=None,
          ws=None, ws_bytes=0, G=0, K=0):
    return lib.ssm_scan_fwd_planned(batch, L, dim, N, io, x, delta, A, B, C, D, z, h0, y,
                                    h_last, ws, ws_bytes, G, K, None)


def test_scan_rejects_bad_arguments(lib):
    assert _scan(lib, batch=-1) == ssm.SSM_ERR_INVALID_ARG
    assert _scan(lib, L=-1) == ssm.SSM_ERR_INVALID_ARG
    assert _scan(lib, io=7) == ssm.SSM_ERR_INVALID_ARG
    assert _scan(lib, x=None) == ssm.SSM_ERR_INVALID_ARG
    assert _scan(lib, A=None) == ssm.SSM_ERR_INVALID_ARG
    assert _scan(lib, y=None) == ssm.SSM_ERR_INVALID_ARG
    assert _scan(lib, y=FAKE) == ssm.SSM_ERR_INVALID_ARG               # y aliases x
    assert _scan(lib, h_last=FAKE) == ssm.SSM_ERR_INVALID_ARG          # h_last aliases x
    assert _scan(lib, N=8) == ssm.SSM_ERR_UNSUPPORTED                   # no kernel, no fallback
    assert _scan(lib, N=24) == ssm.SSM_ERR_UNSUPPORTED
    assert _scan(lib, N=256) == ssm.SSM_ERR_UNSUPPORTED
    assert _scan(lib, G=3) == ssm.SSM_ERR_UNSUPPORTED
    # a chunked plan without workspace
    assert _scan(lib, L=4096, K=4) == ssm.SSM_ERR_WORKSPACE
    need = lib.ssm_scan_workspace_bytes(2, 4096, 64, 16, 1, 4)
    assert need > 0
    assert _scan(lib, L=4096, K=4, ws=ctypes.c_void_p(0x3000), ws_bytes=need - 1) \
        == ssm.SSM_ERR_WORKSPACE


def test_scan_noop_sizes_return_ok_without_launch(lib):
    assert _scan(lib, batch=0) == ssm.SSM_OK
    assert _scan(lib, dim=0) == ssm.SSM_OK
    assert _scan(lib, L=0) == ssm.SSM_OK        # no h_last requested: nothing to do


def test_fused_scan_rejects_bad_arguments(lib):
    W = ctypes.c_void_p(0x4000)

    def fused(batch=2, L=8, dim=64, N=16, io=1, x_raw=FAKE, conv_w=W, d_conv=4, silu=1,
              delta_raw=ctypes.c_void_p(0x6000), y=ctypes.c_void_p(0x2000), G=0):
        return lib.ssm_scan_fwd_fused(batch, L, dim, N, io, x_raw, conv_w, None, d_conv, silu,
                                      delta_raw, None, ctypes.c_void_p(0x7000), FAKE, FAKE,
                                      None, None, None, y, None, None, 0, G, 1, None)
    assert fused(d_conv=0) == ssm.SSM_ERR_INVALID_ARG
    assert fused(d_conv=5) == ssm.SSM_ERR_UNSUPPORTED
    assert fused(silu=2) == ssm.SSM_ERR_INVALID_ARG
    assert fused(conv_w=None) == ssm.SSM_ERR_INVALID_ARG
    assert fused(x_raw=None) == ssm.SSM_ERR_INVALID_ARG
    assert fused(y=W) == ssm.SSM_ERR_INVALID_ARG            # y aliases conv_w
    assert fused(G=16) == ssm.SSM_ERR_UNSUPPORTED           # fused loader needs <= 8 waves
    assert fused(N=8) == ssm.SSM_ERR_UNSUPPORTED
    assert fused(batch=0) == ssm.SSM_OK


def test_scan_variants_reject_bad_arguments(lib):
    def ex(per_channel=1, disc=ssm.SSM_DISC_EULER, batch=2, L=8, G=0, A=FAKE, io=1):
        return lib.ssm_scan_fwd_ex(batch, L, 64, 16, io, FAKE, ctypes.c_void_p(0x6000), A,
                                   per_channel, disc, ctypes.c_void_p(0x7000),
                                   ctypes.c_void_p(0x8000), None, None, None,
                                   ctypes.c_void_p(0x2000), None, None, 0, G, 1, None)
    assert ex(per_channel=2) == ssm.SSM_ERR_INVALID_ARG
    assert ex(per_channel=-1) == ssm.SSM_ERR_INVALID_ARG
    assert ex(disc=2) == ssm.SSM_ERR_INVALID_ARG
    assert ex(A=None) == ssm.SSM_ERR_INVALID_ARG
    assert ex(io=5) == ssm.SSM_ERR_INVALID_ARG
    assert ex(G=16) == ssm.SSM_ERR_UNSUPPORTED              # variants need <= 8 waves
    assert ex(batch=0) == ssm.SSM_OK
    assert ex(L=0) == ssm.SSM_OK


def test_decode_rejects_bad_arguments(lib):
    def dec(batch=2, dim=64, N=16, io=1, h=ctypes.c_void_p(0x5000), x=FAKE,
            y=ctypes.c_void_p(0x2000)):
        return lib.ssm_decode_step(batch, dim, N, io, h, x, FAKE, FAKE, FAKE, FAKE, None,
                                   None, y, None)
    assert dec(batch=-1) == ssm.SSM_ERR_INVALID_ARG
    assert dec(h=None) == ssm.SSM_ERR_INVALID_ARG
    assert dec(y=FAKE) == ssm.SSM_ERR_INVALID_ARG
    assert dec(h=FAKE) == ssm.SSM_ERR_INVALID_ARG
    assert dec(N=4) == ssm.SSM_ERR_UNSUPPORTED
    assert dec(io=2) == ssm.SSM_ERR_INVALID_ARG
    assert dec(batch=0) == ssm.SSM_OK


def test_scan_phase_values(lib):
    """Phase bits 1 and 2 select the launches, 4 the three-pass schedule;
    anything else is rejected before a launch (batch 0 would return OK after
    the check, so a bad phase is seen first)."""
    def phase(ph, batch=0):
        return lib.ssm_scan_fwd_phase(batch, 8, 64, 16, 1, FAKE, ctypes.c_void_p(0x6000), FAKE,
                                      ctypes.c_void_p(0x7000), ctypes.c_void_p(0x8000), None,
                                      None, None, ctypes.c_void_p(0x2000), None, None, 0, 0, 0,
                                      ph, None)
    for bad in (-1, 0, 4, 8, 11):
        assert phase(bad) == ssm.SSM_ERR_INVALID_ARG, bad
    for good in (1, 2, 3, 5, 6, 7):
        assert phase(good) == ssm.SSM_OK, good
    for split in (1, 2, 5, 6):                   # sliced batches take whole scans only
        assert phase(split, batch=65536) == ssm.SSM_ERR_UNSUPPORTED


def test_noalloc_checks_come_first(lib):
    """The allocation-free scan validates like the others and refuses a plan
    whose workspace exceeds its scratch array, all before any HIP call (so
    this runs without a GPU)."""
    def na(batch=2, L=8, dim=64, N=16, io=1, x=FAKE, y=ctypes.c_void_p(0x2000), G=0, K=0):
        return lib.ssm_scan_fwd_noalloc(batch, L, dim, N, io, x, ctypes.c_void_p(0x6000),
                                        FAKE, ctypes.c_void_p(0x7000), ctypes.c_void_p(0x8000),
                                        None, None, None, y, None, G, K, None)
    assert na(batch=-1) == ssm.SSM_ERR_INVALID_ARG
    assert na(x=None) == ssm.SSM_ERR_INVALID_ARG
    assert na(y=FAKE) == ssm.SSM_ERR_INVALID_ARG                  # y aliases x
    assert na(N=8) == ssm.SSM_ERR_UNSUPPORTED
    assert na(G=3) == ssm.SSM_ERR_UNSUPPORTED
    assert na(batch=0) == ssm.SSM_OK
    # 128 chunks of the 262144-step, 4096-channel sequence need 71.3 MB
    assert na(batch=1, L=262144, dim=4096, K=128) == ssm.SSM_ERR_WORKSPACE
    assert lib.ssm_scan_workspace_bytes(1, 262144, 4096, 16, 1, 128) > ssm.SSM_NOALLOC_SCRATCH_BYTES


def test_batch_limits(lib):
    """More than 65535 batch rows: the forward scan slices them (but not when
    its two phases are enqueued apart), the backward refuses; both checks
    come before any launch."""
    assert lib.ssm_scan_fwd_phase(65536, 8, 64, 16, 1, FAKE, ctypes.c_void_p(0x6000), FAKE,
                                  ctypes.c_void_p(0x7000), ctypes.c_void_p(0x8000), None, None,
                                  None, ctypes.c_void_p(0x2000), None, None, 0, 0, 0, 1,
                                  None) == ssm.SSM_ERR_UNSUPPORTED
    p = [ctypes.c_void_p(0x1000 * k) for k in range(1, 20)]
    st = lib.ssm_scan_bwd(65536, 8, 64, 16, 1, p[0], p[1], p[2], 0, ssm.SSM_DISC_ZOH, p[3], p[4],
                          None, None, None, p[5], None, p[6], p[7], p[8], p[9], p[10], None,
                          None, None, p[11], 1 << 40, None)
    assert st == ssm.SSM_ERR_UNSUPPORTED


def test_backward_output_may_not_be_the_workspace(lib):
    p = [ctypes.c_void_p(0x1000 * k) for k in range(1, 20)]
    ws = p[6]                                                    # also passed as dx
    st = lib.ssm_scan_bwd(2, 8, 64, 16, 1, p[0], p[1], p[2], 0, ssm.SSM_DISC_ZOH, p[3], p[4],
                          None, None, None, p[5], None, ws, p[7], p[8], p[9], p[10], None,
                          None, None, ws, 1 << 40, None)
    assert st == ssm.SSM_ERR_INVALID_ARG


def test_ssd_workspace_sizes(lib):
    """The masked-matrix forward's workspace: per 32-step chunk of each batch
    row, C with its states reordered (32 x dstate bf16), B^T (dstate x 32
    bf16) and three 16 x 16 fp32 tiles of C B^T; with segments, also two
    [batch, nseg, dim, dstate] fp32 state arrays and the [batch, nseg,
    nheads] decays; every part 256-byte aligned."""
    def al(v):
        return (v + 255) // 256 * 256

    for B, L, H, N in [(1, 4096, 2, 128), (3, 1000, 5, 64), (2, 1, 1, 128)]:
        nck = (L + 31) // 32
        base = 2 * al(B * nck * 32 * N * 2) + al(B * nck * 3 * 64 * 16)
        assert lib.ssm_ssd_fwd_workspace_bytes(B, L, H, 64, N, 1) == base, (B, L, H, N)
    n4 = lib.ssm_ssd_fwd_workspace_bytes(1, 4096, 2, 64, 128, 4)
    assert n4 == 2 * 1048576 + 393216 + 2 * al(4 * 128 * 128 * 4) + al(4 * 2 * 4)
    assert lib.ssm_ssd_fwd_workspace_bytes(1, 0, 2, 64, 128, 1) == 0
    assert lib.ssm_ssd_fwd_workspace_bytes(-1, 8, 2, 64, 128, 1) == -1
    # too small a workspace is refused before any launch, with or without segments
    for nsplit in (1, 4):
        st = lib.ssm_ssd_fwd_planned(1, 4096, 2, 64, 128, 1, ssm.SSM_DISC_ZOH, FAKE,
                                     ctypes.c_void_p(0x6000), FAKE, ctypes.c_void_p(0x7000),
                                     ctypes.c_void_p(0x8000), None, None, None,
                                     ctypes.c_void_p(0x2000), None, nsplit,
                                     ctypes.c_void_p(0x9000), 16, None)
        assert st == ssm.SSM_ERR_WORKSPACE, nsplit
    st = lib.ssm_ssd_fwd(1, 4096, 2, 64, 128, 1, ssm.SSM_DISC_ZOH, FAKE, ctypes.c_void_p(0x6000),
                         FAKE, ctypes.c_void_p(0x7000), ctypes.c_void_p(0x8000), None, None,
                         None, ctypes.c_void_p(0x2000), None, None, 0, None)
    assert st == ssm.SSM_ERR_WORKSPACE


def test_ssd_backward_rejects_bad_arguments(lib):
    """Every case fails validation before any launch."""
    q = [ctypes.c_void_p(0x1000 * k) for k in range(1, 30)]
    def bwd(disc=ssm.SSM_DISC_ZOH, io=1, N=64, z=None, dz=None, dx=None, ws_bytes=1 << 40):
        return lib.ssm_ssd_bwd(2, 8, 2, 64, N, io, disc, q[0], q[1], q[2], q[3], q[4], None, z,
                               None, q[5], None, dx or q[6], q[7], q[8], q[9], q[10], None, dz,
                               None, q[11], ws_bytes, None)
    assert bwd(disc=2) == ssm.SSM_ERR_INVALID_ARG
    assert bwd(io=7) == ssm.SSM_ERR_INVALID_ARG
    assert bwd(N=24) == ssm.SSM_ERR_UNSUPPORTED
    assert bwd(z=q[12]) == ssm.SSM_ERR_INVALID_ARG             # z without dz
    assert bwd(dx=q[0]) == ssm.SSM_ERR_INVALID_ARG             # dx aliases x
    assert bwd(ws_bytes=16) == ssm.SSM_ERR_WORKSPACE
    assert lib.ssm_ssd_bwd_workspace_bytes(2, 8, 2, 64, 64, 1) > 0
    assert lib.ssm_ssd_bwd_workspace_bytes(-1, 8, 2, 64, 64, 1) == -1


def test_ssd_backward_workspace_by_path(lib):
    """bf16 with 64-channel heads and 64 or 128 states takes the masked-matrix
    backward: its workspace is the fp32 states entering and leaving every
    32-step chunk plus partial sums (dB, dC per group of 16 heads; dD, dA per
    chunk) and a dh0 scratch, each 256-byte aligned.  fp32 I/O and other
    state sizes take the recurrence path (a different layout)."""
    al = lambda v: (v + 255) // 256 * 256
    for B, L, H, N in ((2, 100, 3, 128), (1, 64, 19, 64), (3, 1, 17, 128)):
        K, G, dim = (L + 31) // 32, (H + 15) // 16, H * 64
        want = (2 * al(B * K * dim * N * 4) + 2 * al(B * L * G * N * 4) + al(B * K * dim * 4)
                + al(B * K * H * 4) + al(B * dim * N * 4))
        assert lib.ssm_ssd_bwd_workspace_bytes(B, L, H, 64, N, 1) == want, (B, L, H, N)
        assert lib.ssm_ssd_bwd_workspace_bytes(B, L, H, 64, N, 0) not in (want, 0, -1)
    assert lib.ssm_ssd_bwd_workspace_bytes(2, 100, 3, 64, 32, 1) > 0   # recurrence path


def test_ssd_rejects_bad_arguments(lib):
    """Every case fails validation (or is a no-op) before any launch."""
    def ssd(batch=2, L=8, H=2, P=64, N=128, io=1, disc=ssm.SSM_DISC_ZOH, x=FAKE, A=FAKE,
            y=ctypes.c_void_p(0x2000), h_last=None):
        return lib.ssm_ssd_fwd(batch, L, H, P, N, io, disc, x, ctypes.c_void_p(0x6000), A,
                               ctypes.c_void_p(0x7000), ctypes.c_void_p(0x8000), None, None,
                               None, y, h_last, ctypes.c_void_p(0x9000), 1 << 30, None)
    assert ssd(batch=-1) == ssm.SSM_ERR_INVALID_ARG
    assert ssd(L=-1) == ssm.SSM_ERR_INVALID_ARG
    assert ssd(P=0) == ssm.SSM_ERR_INVALID_ARG
    assert ssd(io=7) == ssm.SSM_ERR_INVALID_ARG
    assert ssd(disc=2) == ssm.SSM_ERR_INVALID_ARG
    assert ssd(io=0) == ssm.SSM_ERR_UNSUPPORTED               # bf16 only
    assert ssd(P=32) == ssm.SSM_ERR_UNSUPPORTED               # heads of 64 channels
    assert ssd(N=16) == ssm.SSM_ERR_UNSUPPORTED               # 64 or 128 states
    assert ssd(H=(1 << 18) + 1) == ssm.SSM_ERR_UNSUPPORTED    # 32-bit chunk offsets
    assert ssd(A=None) == ssm.SSM_ERR_INVALID_ARG
    assert ssd(x=None) == ssm.SSM_ERR_INVALID_ARG
    assert ssd(y=FAKE) == ssm.SSM_ERR_INVALID_ARG             # y aliases x
    assert ssd(h_last=FAKE) == ssm.SSM_ERR_INVALID_ARG        # h_last aliases x
    assert ssd(x=ctypes.c_void_p(0x1001)) == ssm.SSM_ERR_INVALID_ARG  # misaligned
    assert ssd(batch=0) == ssm.SSM_OK
    assert ssd(H=0) == ssm.SSM_OK
    assert ssd(L=0) == ssm.SSM_OK                             # no h_last: nothing to write


def test_decode_variants_reject_bad_arguments(lib):
    def dec(pc=1, disc=ssm.SSM_DISC_EULER, batch=2, N=16, A=FAKE):
        return lib.ssm_decode_step_ex(batch, 64, N, 1, ctypes.c_void_p(0x5000), FAKE,
                                      ctypes.c_void_p(0x6000), A, pc, disc,
                                      ctypes.c_void_p(0x7000), ctypes.c_void_p(0x8000), None,
                                      None, ctypes.c_void_p(0x2000), None)
    assert dec(pc=2) == ssm.SSM_ERR_INVALID_ARG
    assert dec(disc=3) == ssm.SSM_ERR_INVALID_ARG
    assert dec(A=None) == ssm.SSM_ERR_INVALID_ARG
    assert dec(N=24) == ssm.SSM_ERR_UNSUPPORTED
    assert dec(batch=0) == ssm.SSM_OK


def test_plan_and_workspace(lib):
    import torch
    g, k = ssm.scan_plan(4, 4096, 5120)
    assert g in (1, 2, 4, 8, 16) and k >= 1
    assert ssm.scan_workspace_bytes(4, 4096, 5120, nchunks=1) == 0
    # hloc + hin (fp32 per state) + sum of delta (fp64 per channel), per chunk
    n = ssm.scan_workspace_bytes(1, 1000, 100, nchunks=3)
    assert n >= 2 * 3 * 100 * 16 * 4 + 3 * 100 * 8
    # the chunk count is clamped to the sequence length
    assert ssm.scan_workspace_bytes(1, 2, 100, nchunks=50) == \
        ssm.scan_workspace_bytes(1, 2, 100, nchunks=2)
    # the long single sequence is cut into chunks for parallelism
    g3, k3 = ssm.scan_plan(1, 262144, 4096)
    assert k3 > 1 and 262144 / k3 <= 2048   # chunks of at most 2048 steps
    # the cost model's choices on the three measured layer shapes, all in the
    # two-launch schedule: the Mamba-2.8B layer takes 4 chunks (timed equal to
    # 5 within noise, with a third less of x and delta read twice); the long
    # single sequence takes 241 chunks, whose main launch fills 12 whole
    # rounds of five blocks per CU
    assert ssm.scan_plan(4, 4096, 5120, with_phase=True) == (4, 4, 3)
    assert ssm.scan_plan(8, 2048, 1536, with_phase=True) == (4, 5, 3)
    assert ssm.scan_plan(1, 262144, 4096, with_phase=True) == (4, 241, 3)
    # one chunk when the sequence is too short to cut: no schedule to choose
    assert ssm.scan_plan(1, 256, 64, dtype=torch.float32, with_phase=True) == (4, 1, 3)
    lib = ssm.load_library()
    g, k = ctypes.c_int(), ctypes.c_int()
    assert lib.ssm_scan_plan(4, 4096, 5120, 16, ssm.SSM_DTYPE_BF16, ctypes.byref(g),
                             ctypes.byref(k), None) == ssm.SSM_OK and k.value == 4
    with pytest.raises(ValueError):
        ssm.scan_workspace_bytes(-1, 10, 10)


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        ssm.scan_fwd(x, x, torch.zeros(8, 16), torch.zeros(1, 4, 16), torch.zeros(1, 4, 16))
    with pytest.raises(ValueError):
        ssm.decode_step(torch.zeros(1, 8, 16), torch.zeros(1, 8), torch.zeros(1, 8),
                        torch.zeros(8, 16), torch.zeros(1, 16), torch.zeros(1, 16))
