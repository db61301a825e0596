"""The C-ABI library without a GPU: it loads, exports every symbol that
include/pba.h declares, sizes workspaces, and rejects invalid calls with the
documented status codes before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

from pair_biased_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pba.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_ALIGN, ERR_WS, ERR_HIP, ERR_SCRATCH = 0, 1, 2, 3, 4, 5, 6, 7


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail(f"libpba.so is not built ({_lib.LIB_PATH}); run __graft_entry__.build()")
    return _lib.load()


def test_header_declares_the_boundary():
    names = _declared()
    for fn in ("pba_forward", "pba_backward", "pba_backward_workspace_bytes", "pair_weighted_avg",
               "pair_weighted_avg_backward", "pair_weighted_avg_workspace_bytes",
               "pair_weighted_avg_backward_workspace_bytes", "pba_status_string", "pba_abi_version",
               "pba_bias_proj_forward", "pba_bias_proj_backward", "pba_bias_proj_backward_workspace_bytes",
               "pba_local_forward", "pba_local_backward", "pba_local_backward_workspace_bytes"):
        assert fn in names, fn
    assert set(names) == set(_lib.SIGNATURES), (names, sorted(_lib.SIGNATURES))


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name


def test_version_and_status_strings(lib):
    assert lib.pba_abi_version() == 4
    for code in range(8):
        assert lib.pba_status_string(code)
    assert b"unknown" in lib.pba_status_string(99)


def test_workspace_sizes(lib):
    # attention: dA (input dtype) + D (fp32) + partials (fp32 [P,H,N,N])
    for (B, H, N, d, dt) in [(384, 4, 384, 32, 1), (48, 16, 384, 48, 1), (32, 4, 32, 32, 0)]:
        ws = lib.pba_backward_workspace_bytes(B, H, N, d, dt)
        assert ws >= B * H * N * d * (2 if dt else 4) + B * H * N * 4 + H * N * N * 4
        assert ws % 256 == 0
    # B = 1: dS is dBias and goes straight to the output, so no partial plane
    for dt in (1, 0):
        ws = lib.pba_backward_workspace_bytes(1, 16, 768, 24, dt)
        rows = 16 * 768
        assert rows * 24 * (2 if dt else 4) + rows * 4 <= ws < rows * 24 * (2 if dt else 4) + rows * 8 + 1024
        assert ws % 256 == 0
    assert lib.pair_weighted_avg_workspace_bytes(1024, 768, 8, 32, 1) >= 8 * 768 * 768 * 2
    assert lib.pair_weighted_avg_backward_workspace_bytes(1024, 768, 8, 32, 1) >= 1024 * 768 * 8 * 32 * 2
    # invalid sizes give 0
    assert lib.pba_backward_workspace_bytes(0, 4, 384, 32, 1) == 0
    assert lib.pba_backward_workspace_bytes(1, 4, 384, 30, 1) == 0
    assert lib.pair_weighted_avg_workspace_bytes(4, 16, 2, 32, 0) == 0  # fp32 not offered for PWA


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails before use


def _fwd(lib, B=2, H=2, N=64, d=32, dt=1, ptrs=None, mask=None):
    p = [FAKE] * 8 if ptrs is None else ptrs
    return lib.pba_forward(B, H, N, d, dt, p[0], p[1], p[2], p[3], p[4], mask, p[5], p[6], None)


def test_forward_validation(lib):
    assert _fwd(lib, B=0) == ERR_SHAPE
    assert _fwd(lib, N=-3) == ERR_SHAPE
    assert _fwd(lib, d=12) == ERR_UNSUP
    assert _fwd(lib, d=72) == ERR_UNSUP
    assert _fwd(lib, dt=7) == ERR_UNSUP
    for i in range(7):
        ptrs = [FAKE] * 8
        ptrs[i] = None
        assert _fwd(lib, ptrs=ptrs) == ERR_NULL, i
    for i in range(6):
        ptrs = [FAKE] * 8
        ptrs[i] = FAKE + 8
        assert _fwd(lib, ptrs=ptrs) == ERR_ALIGN, i
    assert _fwd(lib, B=1 << 20, H=64, N=4096, d=64) == ERR_SHAPE


def test_backward_validation(lib):
    B, H, N, d = 2, 2, 64, 32
    need = lib.pba_backward_workspace_bytes(B, H, N, d, 1)

    def call(ws=FAKE, wsb=None, null_at=None, misalign_at=None, d_=d):
        p = [FAKE] * 13
        if null_at is not None:
            p[null_at] = None
        if misalign_at is not None:
            p[misalign_at] = FAKE + 4
        return lib.pba_backward(B, H, N, d_, 1, p[0], p[1], p[2], p[3], p[4], None, p[5], p[6], p[7],
                                p[8], p[9], p[10], p[11], p[12], ws, need if wsb is None else wsb, None)

    assert call(d_=20) == ERR_UNSUP
    for i in range(13):
        assert call(null_at=i) == ERR_NULL, i
    assert call(misalign_at=0) == ERR_ALIGN
    assert call(ws=None) == ERR_WS
    assert call(wsb=need - 1) == ERR_WS
    assert call(ws=FAKE + 8) == ERR_ALIGN


def test_backward_noalloc_validation(lib):
    """Every argument check of the allocation-free backward runs before its
    first HIP call, so these run without a GPU."""
    B, H, N, d = 2, 2, 64, 32

    def call(B_=B, N_=N, d_=d, null_at=None, misalign_at=None):
        p = [FAKE] * 13
        if null_at is not None:
            p[null_at] = None
        if misalign_at is not None:
            p[misalign_at] = FAKE + 4
        return lib.pba_backward_noalloc(B_, H, N_, d_, 1, p[0], p[1], p[2], p[3], p[4], None, p[5], p[6],
                                        p[7], p[8], p[9], p[10], p[11], p[12], None)

    assert call(d_=20) == ERR_UNSUP
    assert call(B_=0) == ERR_SHAPE
    for i in range(13):
        assert call(null_at=i) == ERR_NULL, i
    assert call(misalign_at=0) == ERR_ALIGN
    # sizes whose workspace exceeds the static area: rejected before any HIP call
    assert lib.pba_backward_workspace_bytes(1024, H, 768, d, 1) > _lib.NOALLOC_SCRATCH_BYTES
    assert call(B_=1024, N_=768) == ERR_SCRATCH
    assert b"128 MiB" in lib.pba_status_string(ERR_SCRATCH)
    # the triangle workload fits
    assert lib.pba_backward_workspace_bytes(384, 4, 384, 32, 1) <= _lib.NOALLOC_SCRATCH_BYTES
    hdr = open(HEADER).read()
    assert "#define PBA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in hdr
    assert _lib.NOALLOC_SCRATCH_BYTES == 128 << 20


def test_pwa_validation(lib):
    S, N, H, d = 4, 64, 2, 32
    need = lib.pair_weighted_avg_workspace_bytes(S, N, H, d, 1)
    f = lambda dt=1, ws=FAKE, wsb=need, p4=FAKE: lib.pair_weighted_avg(
        S, N, H, d, dt, FAKE, None, FAKE, FAKE, p4, FAKE, ws, wsb, None)
    assert f(dt=0) == ERR_UNSUP
    assert f(p4=None) == ERR_NULL
    assert f(ws=None) == ERR_WS
    assert f(wsb=need - 2) == ERR_WS
    needb = lib.pair_weighted_avg_backward_workspace_bytes(S, N, H, d, 1)
    g = lambda ws=FAKE, wsb=needb, db=FAKE: lib.pair_weighted_avg_backward(
        S, N, H, d, 1, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, db, ws, wsb, None)
    assert g(db=None) == ERR_NULL
    assert g(db=FAKE + 2) == ERR_ALIGN
    assert g(wsb=needb - 1) == ERR_WS


def test_timed_entry_points_validate_like_their_calls(lib):
    """The measurement variants run the same argument checks first and need
    both output pointers; every case here returns before anything touches a GPU."""
    B, H, N, d = 2, 2, 64, 32
    need = lib.pba_backward_workspace_bytes(B, H, N, d, 1)
    p = [FAKE] * 13
    bwd = lambda ws=FAKE, ms=FAKE, n=FAKE, d_=d: lib.pba_backward_timed(
        B, H, N, d_, 1, p[0], p[1], p[2], p[3], p[4], None, p[5], p[6], p[7], p[8], p[9], p[10], p[11], p[12],
        ws, need, None, ms, 4, n)
    assert bwd(d_=20) == ERR_UNSUP
    assert bwd(ws=None) == ERR_WS
    assert bwd(ms=None) == ERR_NULL
    assert bwd(n=None) == ERR_NULL
    S, N2, H2, d2 = 4, 64, 2, 32
    needf = lib.pair_weighted_avg_workspace_bytes(S, N2, H2, d2, 1)
    fwd = lambda ms=FAKE, dt=1: lib.pair_weighted_avg_timed(
        S, N2, H2, d2, dt, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, needf, None, ms, 2, FAKE)
    assert fwd(dt=0) == ERR_UNSUP
    assert fwd(ms=None) == ERR_NULL
    needb = lib.pair_weighted_avg_backward_workspace_bytes(S, N2, H2, d2, 1)
    pb = lambda ws=FAKE, ms=FAKE: lib.pair_weighted_avg_backward_timed(
        S, N2, H2, d2, 1, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, needb, None, ms, 8, FAKE)
    assert pb(ws=None) == ERR_WS
    assert pb(ms=None) == ERR_NULL


def test_bias_proj_workspace_sizes(lib):
    # one partial record of 16 c + 16 floats per backward workgroup, at most 256 workgroups
    for N, H, c in [(384, 4, 128), (768, 16, 128), (5, 3, 32), (64, 16, 64)]:
        ws = lib.pba_bias_proj_backward_workspace_bytes(N, H, c, 1)
        rec = (16 * c + 16) * 4
        assert ws > 0 and ws % rec == 0 and ws // rec <= 256
    # the record count follows N and c only, not H
    assert (lib.pba_bias_proj_backward_workspace_bytes(768, 16, 128, 1)
            == lib.pba_bias_proj_backward_workspace_bytes(768, 1, 128, 1))
    assert lib.pba_bias_proj_backward_workspace_bytes(768, 16, 128, 0) == 0   # bf16 only
    assert lib.pba_bias_proj_backward_workspace_bytes(768, 17, 128, 1) == 0   # H <= 16
    assert lib.pba_bias_proj_backward_workspace_bytes(768, 4, 96, 1) == 0     # c in {32, 64, 128}
    assert lib.pba_bias_proj_backward_workspace_bytes(0, 4, 128, 1) == 0
    assert lib.pba_bias_proj_backward_workspace_bytes(5000, 4, 128, 1) == 0   # z too large


def test_bias_proj_validation(lib):
    N, H, c = 64, 4, 128

    def f(N_=N, H_=H, c_=c, dt=1, eps=1e-5, p=None):
        z, gamma, beta, w, bias = p or [FAKE] * 5
        return lib.pba_bias_proj_forward(N_, H_, c_, dt, z, gamma, beta, w, eps, bias, None)

    assert f(dt=0) == ERR_UNSUP
    assert f(H_=17) == ERR_UNSUP
    assert f(c_=48) == ERR_UNSUP
    assert f(N_=0) == ERR_SHAPE
    assert f(eps=0.0) == ERR_SHAPE
    assert f(eps=float("nan")) == ERR_SHAPE
    assert f(eps=float("inf")) == ERR_SHAPE
    for i in range(5):
        p = [FAKE] * 5
        p[i] = None
        assert f(p=p) == ERR_NULL, i
    p = [FAKE] * 5
    p[0] = FAKE + 8  # z must be 16-byte aligned
    assert f(p=p) == ERR_ALIGN
    p = [FAKE] * 5
    p[1] = FAKE + 4  # gamma must be 16-byte aligned too
    assert f(p=p) == ERR_ALIGN
    need = lib.pba_bias_proj_backward_workspace_bytes(N, H, c, 1)

    def b(ws=FAKE, wsb=need, null_at=None, misalign=None, dt=1):
        p = [FAKE] * 9
        if null_at is not None:
            p[null_at] = None
        if misalign is not None:
            p[misalign[0]] = FAKE + misalign[1]
        return lib.pba_bias_proj_backward(N, H, c, dt, p[0], p[1], p[2], p[3], 1e-5, p[4], p[5], p[6], p[7],
                                          p[8], ws, wsb, None)

    assert b(dt=0) == ERR_UNSUP
    for i in range(9):
        assert b(null_at=i) == ERR_NULL, i
    assert b(misalign=(4, 8)) == ERR_ALIGN   # dbias
    assert b(misalign=(5, 8)) == ERR_ALIGN   # dz
    assert b(misalign=(8, 4)) == ERR_ALIGN   # dw
    assert b(ws=None) == ERR_WS
    assert b(wsb=need - 4) == ERR_WS
    assert b(ws=FAKE + 8) == ERR_ALIGN
    ms = lambda m=FAKE, n=FAKE: lib.pba_bias_proj_forward_timed(N, H, c, 1, FAKE, FAKE, FAKE, FAKE, 1e-5, FAKE,
                                                                None, m, 1, n)
    assert ms(m=None) == ERR_NULL and ms(n=None) == ERR_NULL
    mb = lambda ws=FAKE, m=FAKE: lib.pba_bias_proj_backward_timed(
        N, H, c, 1, FAKE, FAKE, FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE, FAKE, FAKE, ws, need, None, m, 2, FAKE)
    assert mb(ws=None) == ERR_WS and mb(m=None) == ERR_NULL


def test_local_attention_validation(lib):
    B, H, N, d = 2, 2, 100, 32
    need = lib.pba_local_backward_workspace_bytes(B, H, N, d, 1)
    assert need >= B * H * N * d * 2 + B * H * N * 8 + H * 4 * 32 * 128 * 4
    assert lib.pba_local_backward_workspace_bytes(B, H, N, 40, 1) == 0   # d <= 32
    assert lib.pba_local_backward_workspace_bytes(B, H, N, d, 0) == 0    # bf16 only
    assert lib.pba_local_backward_workspace_bytes(B, H, N, 12, 1) == 0   # multiple of 8

    def f(dt=1, d_=d, p=None):
        q, k, v, g, bias, out, lse = p or [FAKE] * 7
        return lib.pba_local_forward(B, H, N, d_, dt, q, k, v, g, bias, None, out, lse, None)

    assert f(dt=0) == ERR_UNSUP and f(d_=64) == ERR_UNSUP
    for i in range(7):
        p = [FAKE] * 7
        p[i] = None
        assert f(p=p) == ERR_NULL, i
    p = [FAKE] * 7
    p[4] = FAKE + 8
    assert f(p=p) == ERR_ALIGN

    def b(ws=FAKE, wsb=need, null_at=None):
        p = [FAKE] * 13
        if null_at is not None:
            p[null_at] = None
        return lib.pba_local_backward(B, H, N, d, 1, p[0], p[1], p[2], p[3], p[4], None, p[5], p[6], p[7],
                                      p[8], p[9], p[10], p[11], p[12], ws, wsb, None)

    for i in range(13):
        assert b(null_at=i) == ERR_NULL, i
    assert b(ws=None) == ERR_WS and b(wsb=need - 1) == ERR_WS and b(ws=FAKE + 8) == ERR_ALIGN
    tb = lambda m=FAKE: lib.pba_local_backward_timed(B, H, N, d, 1, *([FAKE] * 5), None, *([FAKE] * 8), FAKE,
                                                    need, None, m, 4, FAKE)
    assert tb(m=None) == ERR_NULL


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    import pair_biased_attention_amd as pba
    x = torch.zeros(1, 1, 8, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pba.pba_forward(x, x, x, x, torch.zeros(1, 8, 8, dtype=torch.bfloat16))
