"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: per output tensor, max |gpu - oracle| <= tol * max |oracle| with
tol = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (fp32 accumulation),
each tensor measured against its own largest oracle value; masked positions
and fully-masked rows bit-exact.  Every element is compared, the full-size
triangle, Pairformer, diffusion-copy and pair-weighted-average workloads
included.  Only the MSA row attention workload (4.8e9 score elements) is
compared on sampled batch rows (each batch row is independent) and on sampled
bias-gradient rows, which the oracle sums over every batch row.
"""
from __future__ import annotations

import ctypes
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, assert_close, bits_to_f64, check_all, log, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pair_biased_attention_amd._lib as L
    L.load()  # fails loudly if the library is missing


import pair_biased_attention_amd as pba  # noqa: E402


# ----------------------------------------------------------------- helpers

def _attn_case(B, H, N, d, dtype, mask, seed):
    cfg = workloads.AttnConfig("case", B=B, H=H, N=N, d=d, dtype=dtype, mask=mask, seed=seed)
    return workloads.attention_inputs(cfg)


def _run_attn(inp, dtype):
    dev = {n: to_dev(inp[n], dtype) for n in ("q", "k", "v", "g", "bias", "dout")}
    km = None if inp["key_mask"] is None else to_dev(inp["key_mask"], dtype)
    out, lse = pba.pba_forward(dev["q"], dev["k"], dev["v"], dev["g"], dev["bias"], km)
    grads = pba.pba_backward(dev["q"], dev["k"], dev["v"], dev["g"], dev["bias"], km, out, lse, dev["dout"])
    torch.cuda.synchronize()
    res = {"out": to_f64(out), "lse": lse.cpu().numpy().astype(np.float64)}
    res.update({k: to_f64(v) for k, v in grads.items()})
    return res


def _check_attn_full(inp, res, dtype, tag, zero_ds=False):
    """Every element of every output against the oracle, each tensor against
    its own max |ref|.

    zero_ds: the oracle's dS is identically zero (a single kept key: its row
    of P is exactly 1, so dP - D vanishes).  dq, dk and dbias are then zero
    up to rounding, while the kernels form D = rowsum(dO * O) from O in the
    storage dtype and so carry an absolute error of order eps * |dO| |O|;
    only in that case is their bar taken relative to max |dv|, the size of
    the products that cancel.
    """
    tol = TOL[dtype]
    O, L = oracle.attention_forward(inp["q64"], inp["k64"], inp["v64"], inp["g64"], inp["bias64"], inp["key_mask"])
    gr = oracle.attention_backward(inp["q64"], inp["k64"], inp["v64"], inp["g64"], inp["bias64"],
                                   inp["key_mask"], inp["dout64"])
    pairs = {"out": (res["out"], O), "lse": (res["lse"], L)}
    pairs.update({n: (res[n], gr[n]) for n in ("dq", "dk", "dv", "dg", "dbias")})
    floors = None
    if zero_ds:
        assert all(np.max(np.abs(gr[n])) < 1e-12 * np.max(np.abs(gr["dv"])) for n in ("dq", "dk", "dbias"))
        floor = float(np.max(np.abs(gr["dv"])))
        floors = {n: floor for n in ("dq", "dk", "dbias")}

    check_all(tag, pairs, tol, floors)
    return gr


# ----------------------------------------------------------------- attention, small

SMALL_ATTN = [
    # B, H, N, d, dtype, mask
    (3, 2, 200, 32, "bf16", "tail:7"),       # ragged N, tail mask, several key blocks
    (3, 2, 380, 32, "bf16", "tail:9"),       # six query blocks, N % 8 != 0: dBias slab in registers, all block pairs
    (2, 3, 130, 24, "bf16", "random:10"),    # d padded 24 -> 32
    (2, 2, 96, 48, "bf16", "none"),          # d = 48 (three 16-wide column tiles)
    (2, 2, 77, 64, "bf16", "random:5"),
    (2, 2, 70, 8, "bf16", "none"),
    (1, 2, 150, 16, "bf16", "random:4"),     # B = 1: dS is stored straight into the bias gradient
    (1, 2, 97, 64, "bf16", "tail:5"),        # the same in the 64-wide template, ragged N
    (1, 3, 90, 32, "f32", "random:6"),       # the same on the fp32 path
    (40, 1, 64, 32, "bf16", "tail:3"),       # several batch chunks and partials
    (4, 2, 100, 32, "f32", "random:9"),
    (2, 2, 65, 48, "f32", "none"),
    (3, 1, 33, 64, "f32", "random:2"),
    # small grids (B H ceil(N/64) < 512) with N % 8 == 0 and d <= 32 take the
    # key-split forward and key-split dQ tiles: four waves per 16-query tile,
    # each a range of key blocks
    (1, 3, 328, 24, "bf16", "random:12"),    # six blocks over four waves (1, 2, 1, 2), ragged last block
    (2, 2, 1000, 32, "bf16", "tail:40"),     # sixteen blocks, the masked tail inside the last wave's range
    (1, 1, 136, 16, "bf16", "none"),         # three blocks: wave 0 has no keys
    (1, 2, 256, 32, "bf16", "tail:64"),      # one block per wave, the last wave's block wholly masked
    (1, 2, 2048, 8, "bf16", "random:30"),    # 32 blocks, d = 8
    (2, 2, 264, 32, "bf16", "random:17"),    # the same split for dQ beside dK/dV tiles with the dBias slab in LDS
    # a dBias slab too large for two workgroups per CU: separate dK/dV and dQ
    # launches.  384 < N <= 768 at d <= 32 (N % 8 == 0): eight-wave dK/dV
    # workgroups in 128-query steps with the slab in registers; at d > 32 the
    # eight-wave 64-query tiles beside an LDS slab
    (3, 2, 456, 32, "bf16", "tail:11"),      # four steps per row, the last one 72 queries
    (4, 2, 520, 32, "bf16", "random:9"),     # five steps, the last one 8 queries
    (3, 3, 640, 16, "bf16", "tail:30"),      # five full steps, d = 16
    (2, 2, 768, 24, "bf16", "none"),         # six steps, d = 24
    (24, 2, 448, 32, "bf16", "tail:13"),     # several batch chunks of a few rows each
    (8, 2, 392, 32, "bf16", "tail:3"),       # the smallest N of the eight-wave path: the last step 8 queries
    (4, 2, 300, 64, "bf16", "random:13"),    # d = 64, N % 8 != 0 (element-wise bias loads)
    (2, 3, 520, 48, "bf16", "tail:20"),      # d = 48 in the 64-wide tile, slab 72 KB (159 KB with the tiles)
    (2, 2, 600, 64, "bf16", "none"),         # slab 80 KB: too large beside the eight-wave tiles, four-wave tile
    # grids of >= 512 (b, h) workgroups take the K/V-resident forward kernel;
    # with N <= 384, N % 8 == 0 and d <= 32 the dK/dV tiles take 128-query
    # steps with LDS-destination staging
    (128, 4, 200, 24, "bf16", "tail:7"),     # ragged N, padded d, idle waves past N; two steps per row
    (32, 4, 264, 32, "bf16", "random:17"),   # three steps per row, the last one 8 queries
    (64, 4, 128, 16, "bf16", "tail:5"),      # one step per row, d = 16
    (48, 4, 248, 24, "bf16", "none"),        # two steps per row, the second ragged
    (256, 2, 8, 8, "bf16", "none"),          # N = 8, d = 8: one step, 24 of the tile's 32 keys past N
    (64, 8, 136, 48, "bf16", "random:5"),    # d = 48 in the 64-wide template
    (515, 2, 264, 24, "bf16", "random:17"),  # many (b, h): the second query block's last two waves without rows
    (256, 4, 320, 32, "bf16", "tail:21"),    # five full key blocks, three 128-query steps (the last one 64)
]


@pytest.mark.parametrize("B,H,N,d,dtype,mask", SMALL_ATTN)
def test_attention_small(B, H, N, d, dtype, mask):
    log(f"attention small B={B} H={H} N={N} d={d} {dtype} mask={mask}")
    inp = _attn_case(B, H, N, d, dtype, mask, seed=100 + N + d)
    res = _run_attn(inp, dtype)
    gr = _check_attn_full(inp, res, dtype, f"small[{B},{H},{N},{d},{dtype}]")
    if inp["key_mask"] is not None:
        dead = inp["key_mask"] == 0
        assert np.all(res["dk"][:, :, dead] == 0) and np.all(res["dv"][:, :, dead] == 0)
        assert np.all(res["dbias"][:, :, dead] == 0)
        assert np.all(gr["dk"][:, :, dead] == 0)


# ----------------------------------------------------------------- attention, full workloads

def _sample_rows(N):
    """Query rows for the sampled bias-gradient check: the first and last row,
    and one row inside every 64-query block at a varying offset."""
    rows = {0, 1, N - 1}
    for qb in range((N + 63) // 64):
        rows.add(min(N - 1, 64 * qb + (37 * qb + 5) % 64))
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["tiny_fp32", "tri_attn_n384", "pairformer_apb", "dit_apb_x48"])
def test_attention_workload(name):
    """Every element of every output at the full workload size."""
    cfg = workloads.CONFIGS[name]
    dtype = cfg.dtype
    log(f"attention workload {name}: B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} {dtype} mask={cfg.mask}")
    inp = workloads.attention_inputs(cfg)
    res = _run_attn(inp, dtype)
    log(f"{name}: kernels done, oracle on every element")
    _check_attn_full(inp, res, dtype, name)
    if inp["key_mask"] is not None:
        dead = inp["key_mask"] == 0
        assert np.all(res["dk"][:, :, dead] == 0) and np.all(res["dv"][:, :, dead] == 0)
        assert np.all(res["dbias"][:, :, dead] == 0)


def test_msa_row_attention_workload():
    """MSA row attention (B = 1024 rows, N = 768, H = 8): 4.8e9 score
    elements, so batch rows and bias-gradient rows are sampled."""
    cfg = workloads.CONFIGS["msa_row_attn"]
    dtype = cfg.dtype
    tol = TOL[dtype]
    log(f"attention workload msa_row_attn: B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} {dtype} mask={cfg.mask}")
    inp = workloads.attention_inputs(cfg)
    res = _run_attn(inp, dtype)
    # every batch row is independent: compare a sample of rows completely
    bs = np.array(sorted({0, 1, 255, 256, cfg.B // 2 + 3, 777, cfg.B - 2, cfg.B - 1}))
    sub = {n: inp[n + "64"][bs] for n in ("q", "k", "v", "g", "dout")}
    O, L = oracle.attention_forward(sub["q"], sub["k"], sub["v"], sub["g"], inp["bias64"], inp["key_mask"])
    gr = oracle.attention_backward(sub["q"], sub["k"], sub["v"], sub["g"], inp["bias64"], inp["key_mask"], sub["dout"])
    # bias gradient: sampled query rows, summed by the oracle over every batch row
    rows = _sample_rows(cfg.N)
    grr = oracle.attention_backward(inp["q64"][:, :, rows], inp["k64"], inp["v64"], inp["g64"][:, :, rows],
                                    inp["bias64"][:, rows], inp["key_mask"], inp["dout64"][:, :, rows])
    pairs = {"out": (res["out"][bs], O), "lse": (res["lse"][bs], L)}
    pairs.update({n: (res[n][bs], gr[n]) for n in ("dq", "dk", "dv", "dg")})
    pairs["dbias_rows"] = (res["dbias"][:, rows], grr["dbias"])
    check_all("msa_row_attn", pairs, tol)
    dead = inp["key_mask"] == 0
    assert np.all(res["dk"][:, :, dead] == 0) and np.all(res["dv"][:, :, dead] == 0)
    assert np.all(res["dbias"][:, :, dead] == 0)


# ----------------------------------------------------------------- edge cases

def test_fully_masked_keys_and_single_key():
    log("edge: fully masked and single kept key")
    for dtype in ("bf16", "f32"):
        inp = _attn_case(2, 2, 40, 32, dtype, "none", seed=5)
        inp["key_mask"] = np.zeros(40, np.uint8)
        res = _run_attn(inp, dtype)
        assert np.all(res["out"] == 0) and np.all(np.isneginf(res["lse"]))
        for n in ("dq", "dk", "dv", "dg", "dbias"):
            assert np.all(res[n] == 0), (dtype, n)
        km = np.zeros(40, np.uint8)
        km[17] = 1
        inp["key_mask"] = km
        res = _run_attn(inp, dtype)
        _check_attn_full(inp, res, dtype, f"single-key {dtype}", zero_ds=True)


# Two keys, bf16: dS = P1 P2 (dP1 - dP2) is a small difference of large terms,
# so the bf16 rounding of the backward's storage-type operands is amplified:
# dA = dO * sigmoid(G) enters dP = dA V^T as a bf16 matrix-core operand, and O
# (stored in bf16) enters D = rowsum(dO * O).  In fp64 with exactly those two
# roundings and nothing else, dq moves by 1.0e-1 of max|dq| here (7.1e-2 from
# dA alone, 7.8e-2 from O alone), which is what the kernels measure.
_ILL_CONDITIONED = pytest.mark.xfail(
    reason="two-key softmax: bf16 rounding of dA (an MFMA operand) and of the stored O, amplified by the "
           "cancellation in dS, moves dq, dk, dbias past 2e-2", strict=False)
TINY = [(B, H, N, d, dt) for (B, H, N, d) in [(1, 1, 1, 8), (1, 1, 2, 8), (2, 1, 3, 16), (1, 3, 17, 64)]
        for dt in ("bf16", "f32")]


@pytest.mark.parametrize("B,H,N,d,dtype", [
    pytest.param(*c, marks=_ILL_CONDITIONED) if (c[2] == 2 and c[4] == "bf16") else c for c in TINY])
def test_tiny_sizes(B, H, N, d, dtype):
    log(f"edge: tiny B={B} H={H} N={N} d={d} {dtype}")
    inp = _attn_case(B, H, N, d, dtype, "none", seed=9)
    res = _run_attn(inp, dtype)
    # N = 1: the one key is the single kept key, so dS is exactly 0
    _check_attn_full(inp, res, dtype, f"tiny[{B},{H},{N},{d},{dtype}]", zero_ds=N == 1)


def test_reduction_to_plain_attention_on_gpu():
    """bias = 0, G = 40 turns the kernel into plain attention; compare with a
    float32 CPU attention computed by PyTorch's own routine."""
    log("special: bias 0, gate 40 vs torch scaled_dot_product_attention (fp32, CPU)")
    inp = _attn_case(3, 2, 150, 32, "bf16", "random:6", seed=21)
    inp["g"] = workloads.bf16_round_bits(np.full(inp["q"].shape, 40.0, np.float32))
    inp["bias"] = workloads.bf16_round_bits(np.zeros(inp["bias"].shape, np.float32))
    res = _run_attn(inp, "bf16")
    q, k, v = (torch.from_numpy(bits_to_f64(inp[n], "bf16")).float() for n in ("q", "k", "v"))
    mask = torch.from_numpy(inp["key_mask"] != 0).view(1, 1, 1, -1).expand(3, 2, 150, 150)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask).double().numpy()
    assert_close("plain attention", res["out"], ref, TOL["bf16"])


def test_zero_query_key_attention_equals_pwa_on_gpu():
    """Q = K = 0: the attention kernels and the pair-weighted-average kernels
    compute the same function (on transposed layouts)."""
    log("special: attention with Q=K=0 vs pair-weighted average")
    S, N, H, d = 4, 130, 2, 32
    pin = workloads.pwa_inputs(workloads.PwaConfig("eq", S=S, N=N, H=H, d=d, dtype="bf16", mask="none", seed=33))
    t = lambda x: np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))
    z = np.zeros((S, H, N, d), np.uint16)
    ainp = {"q": z, "k": z, "v": t(pin["v"]), "g": t(pin["g"]), "bias": pin["b"], "dout": t(pin["dout"]),
            "key_mask": None}
    ares = _run_attn(ainp, "bf16")
    pres = _run_pwa(pin)
    tol = TOL["bf16"]
    assert_close("Q=K=0 out", t(pres["out"]), ares["out"], tol)
    assert_close("Q=K=0 dv", t(pres["dv"]), ares["dv"], tol)
    assert_close("Q=K=0 dg", t(pres["dg"]), ares["dg"], tol)
    assert_close("Q=K=0 db", pres["db"], ares["dbias"], tol)


# ----------------------------------------------------------------- determinism and guard bands

def test_backward_is_bitwise_deterministic():
    log("determinism: two identical attention backward and PWA backward calls")
    inp = _attn_case(64, 4, 384, 32, "bf16", "tail:19", seed=77)
    r1 = _run_attn(inp, "bf16")
    r2 = _run_attn(inp, "bf16")
    diff = [n for n in r1 if not np.array_equal(r1[n], r2[n], equal_nan=True)]
    assert not diff, f"attention outputs differ between identical calls: {diff}"
    pin = workloads.pwa_inputs(workloads.PwaConfig("det", S=16, N=256, H=2, d=32, dtype="bf16", mask="none", seed=3))
    p1, p2 = _run_pwa(pin), _run_pwa(pin)
    diff = [n for n in p1 if not np.array_equal(p1[n], p2[n])]
    assert not diff, f"pwa outputs differ between identical calls: {diff}"


def test_outputs_stay_inside_their_buffers():
    """Raw C-ABI call with every output placed inside a larger canary-filled buffer."""
    log("guard bands: raw pba_forward / pba_backward")
    import pair_biased_attention_amd._lib as L
    lib = L.load()
    B, H, N, d = 3, 2, 100, 24
    inp = _attn_case(B, H, N, d, "bf16", "random:5", seed=8)
    dev = {n: to_dev(inp[n], "bf16") for n in ("q", "k", "v", "g", "bias", "dout")}
    km = to_dev(inp["key_mask"], "bf16")
    G = 4096  # guard elements on each side (16-byte aligned offsets)
    canary = -12352.0  # exactly representable in bf16 and fp32

    def guarded(n_elem, dtype):
        buf = torch.full((n_elem + 2 * G,), canary, dtype=dtype, device="cuda")
        return buf, buf[G:G + n_elem]

    nt = B * H * N * d
    bufs = {n: guarded(nt, torch.bfloat16) for n in ("out", "dq", "dk", "dv", "dg")}
    bufs["dbias"] = guarded(H * N * N, torch.bfloat16)
    bufs["lse"] = guarded(B * H * N, torch.float32)
    wsb = lib.pba_backward_workspace_bytes(B, H, N, d, 1)
    p = lambda t: t.data_ptr()
    st = lib.pba_forward(B, H, N, d, 1, p(dev["q"]), p(dev["k"]), p(dev["v"]), p(dev["g"]), p(dev["bias"]),
                         p(km), p(bufs["out"][1]), p(bufs["lse"][1]), None)
    assert st == 0
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    st = lib.pba_backward(B, H, N, d, 1, p(dev["q"]), p(dev["k"]), p(dev["v"]), p(dev["g"]), p(dev["bias"]),
                          p(km), p(bufs["out"][1]), p(bufs["lse"][1]), p(dev["dout"]), p(bufs["dq"][1]),
                          p(bufs["dk"][1]), p(bufs["dv"][1]), p(bufs["dg"][1]), p(bufs["dbias"][1]),
                          p(ws), wsb, None)
    assert st == 0
    torch.cuda.synchronize()
    for n, (buf, _) in bufs.items():
        head, tail = buf[:G].float().cpu(), buf[-G:].float().cpu()
        assert torch.all(head == canary) and torch.all(tail == canary), n
    O, _ = oracle.attention_forward(inp["q64"], inp["k64"], inp["v64"], inp["g64"], inp["bias64"], inp["key_mask"])
    assert_close("guarded out", to_f64(bufs["out"][1]).reshape(O.shape), O, TOL["bf16"])


# ----------------------------------------------------------------- pair-weighted average

def _run_pwa(inp):
    dev = {n: to_dev(inp[n], "bf16") for n in ("b", "v", "g", "dout")}
    km = None if inp["key_mask"] is None else to_dev(inp["key_mask"], "bf16")
    out, lse = pba.pair_weighted_avg(dev["b"], dev["v"], dev["g"], km)
    grads = pba.pair_weighted_avg_backward(dev["b"], dev["v"], dev["g"], km, out, lse, dev["dout"])
    torch.cuda.synchronize()
    res = {"out": to_f64(out), "lse": lse.cpu().numpy().astype(np.float64)}
    res.update({k: to_f64(v) for k, v in grads.items()})
    return res


SMALL_PWA = [
    # S, N, H, d, mask
    (6, 200, 2, 32, "none"),
    (5, 90, 3, 64, "random:7"),
    (9, 300, 2, 24, "tail:11"),
    (3, 257, 1, 48, "none"),
    (1, 64, 2, 8, "none"),
    # N % 8 == 0 with a key mask (16-byte row kernels, masked keys), and
    # N > 512 with a partial last 64-chunk round
    (4, 136, 2, 32, "random:9"),
    (2, 520, 1, 16, "tail:5"),
    # N % 8 == 0 with channels padded to 64, an odd head count (a pair with
    # one head) and ragged column and row tiles
    (3, 136, 3, 64, "random:5"),
    (5, 200, 2, 48, "none"),
    # more product tiles (65 column tiles x 2 heads x 2 pairs = 260) than the
    # persistent forward's workgroups, so some walk two tiles, one of them the
    # empty fourth head of an odd count; ragged last column and row tiles
    (517, 136, 3, 32, "random:9"),
]


@pytest.mark.parametrize("S,N,H,d,mask", SMALL_PWA)
def test_pwa_small(S, N, H, d, mask):
    log(f"pwa small S={S} N={N} H={H} d={d} mask={mask}")
    inp = workloads.pwa_inputs(workloads.PwaConfig("case", S=S, N=N, H=H, d=d, dtype="bf16", mask=mask,
                                                   seed=200 + N))
    res = _run_pwa(inp)
    tol = TOL["bf16"]
    O, L = oracle.pwa_forward(inp["b64"], inp["v64"], inp["g64"], inp["key_mask"])
    gr = oracle.pwa_backward(inp["b64"], inp["v64"], inp["g64"], inp["key_mask"], inp["dout64"])
    pairs = {"out": (res["out"], O), "lse": (res["lse"], L)}
    pairs.update({n: (res[n], gr[n]) for n in ("dv", "dg", "db")})
    check_all(f"pwa[{S},{N},{H},{d}]", pairs, tol)
    if inp["key_mask"] is not None:
        dead = inp["key_mask"] == 0
        assert np.all(res["dv"][:, dead] == 0) and np.all(res["db"][:, :, dead] == 0)


def test_pwa_workload():
    """Every element of the pair-weighted average at the full workload size.

    The oracle runs over chunks of MSA rows (each row's out, dv and dg depend
    on that row alone).  db is the sum of the chunks' db: for fixed weights w,
    db = w * (dw - sum_j w * dw) is linear in dw, and dw is a sum over rows.
    """
    cfg = workloads.CONFIGS["msa_pwa"]
    log(f"pwa workload: S={cfg.S} N={cfg.N} H={cfg.H} d={cfg.d}")
    inp = workloads.pwa_inputs(cfg, with_f64=False)
    dev = {n: to_dev(inp[n], "bf16") for n in ("b", "v", "g", "dout")}
    out, lse = pba.pair_weighted_avg(dev["b"], dev["v"], dev["g"], None)
    grads = pba.pair_weighted_avg_backward(dev["b"], dev["v"], dev["g"], None, out, lse, dev["dout"])
    torch.cuda.synchronize()
    tol = TOL["bf16"]
    f64 = lambda x: bits_to_f64(x, "bf16")
    b64 = f64(inp["b"])
    worst = {}
    db_ref = np.zeros_like(b64)
    step = 128
    for s0 in range(0, cfg.S, step):
        s1 = min(cfg.S, s0 + step)
        v_s, g_s, do_s = f64(inp["v"][s0:s1]), f64(inp["g"][s0:s1]), f64(inp["dout"][s0:s1])
        O, L = oracle.pwa_forward(b64, v_s, g_s, None)
        gr = oracle.pwa_backward(b64, v_s, g_s, None, do_s)
        db_ref += gr["db"]
        pairs = {"out": (to_f64(out[s0:s1]), O), "dv": (to_f64(grads["dv"][s0:s1]), gr["dv"]),
                 "dg": (to_f64(grads["dg"][s0:s1]), gr["dg"])}
        if s0 == 0:
            pairs["lse"] = (lse.cpu().numpy().astype(np.float64), L)
        # errors are measured against the whole tensor's max |ref| below;
        # keep each chunk's worst error and max |ref|
        for n, (got, ref) in pairs.items():
            assert np.array_equal(np.isfinite(got), np.isfinite(ref)), n
            e = float(np.max(np.abs(got - ref)))
            m = float(np.max(np.abs(ref)))
            pe, pm = worst.get(n, (0.0, 0.0))
            worst[n] = (max(pe, e), max(pm, m))
        log(f"msa_pwa rows {s0}..{s1 - 1}: " + " ".join(f"{n}={e / m:.2e}" for n, (e, m) in worst.items()))
    e_db = float(np.max(np.abs(to_f64(grads["db"]) - db_ref)))
    worst["db"] = (e_db, float(np.max(np.abs(db_ref))))
    log("msa_pwa: " + " ".join(f"{n}={e / m:.2e}" for n, (e, m) in worst.items()))
    for n, (e, m) in worst.items():
        assert e <= tol * m, f"msa_pwa {n}: max|err| = {e:.3e} > {tol:.1e} * {m:.3e}"
