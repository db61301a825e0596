"""GPU parity of the pair-bias projection bias = Linear(LayerNorm(z)) (HIP path
through the C ABI) against the fp64 oracle in ``oracle/bias_proj_oracle.py``.

Bar: per output tensor, max |gpu - oracle| <= 2e-2 * max |oracle| (bf16 z,
bias, dbias and dz; the products take bf16 operands and accumulate in fp32).
Every element is compared, at the small sizes and at both full workloads:
the oracle finishes the full Pairformer size (z [768, 768, 128]) in seconds.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, check_all, log, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pair_biased_attention_amd._lib as L
    L.load()  # fails loudly if the library is missing


import pair_biased_attention_amd as pba  # noqa: E402

EPS = oracle.BIAS_PROJ_EPS


def _dev(inp):
    d = {"z": to_dev(inp["z"], "bf16"), "dbias": to_dev(inp["dbias"], "bf16")}
    d.update({n: torch.from_numpy(inp[n]).cuda() for n in ("gamma", "beta", "w")})
    return d


def _run(inp):
    d = _dev(inp)
    bias = pba.pba_bias_proj_forward(d["z"], d["gamma"], d["beta"], d["w"], EPS)
    gr = pba.pba_bias_proj_backward(d["z"], d["gamma"], d["beta"], d["w"], d["dbias"], EPS)
    torch.cuda.synchronize()
    res = {"bias": to_f64(bias)}
    res.update({k: to_f64(v) for k, v in gr.items()})
    return res


def _check(inp, res, tag):
    args = (inp["z64"], inp["gamma64"], inp["beta64"], inp["w64"])
    ref = {"bias": oracle.bias_projection_forward(*args, eps=EPS)}
    ref.update(oracle.bias_projection_backward(*args, inp["dbias64"], eps=EPS))
    check_all(tag, {n: (res[n], ref[n]) for n in ("bias", "dz", "dgamma", "dbeta", "dw")}, TOL["bf16"])
    return ref


SMALL = [
    # N, H, c
    (37, 3, 128),    # N*N = 1369: a ragged last tile of 9 positions
    (16, 16, 64),    # H = 16 fills the head axis of the products
    (50, 8, 32),     # one 32-channel slice
    (23, 1, 128),    # a single head
    (130, 16, 128),  # 1057 tiles over 89 backward workgroups, ragged tail of 4
    (1, 4, 128),     # a single position
    (3, 5, 64),      # fewer positions than one tile
]


@pytest.mark.parametrize("N,H,c", SMALL)
def test_bias_proj_small(N, H, c):
    log(f"bias projection small N={N} H={H} c={c}")
    inp = workloads.bias_proj_inputs(workloads.ProjConfig("case", N=N, H=H, c=c, seed=300 + N + H + c))
    _check(inp, _run(inp), f"proj[{N},{H},{c}]")


@pytest.mark.parametrize("name", ["bias_proj_tri_n384", "bias_proj_pairformer"])
def test_bias_proj_workload(name):
    cfg = workloads.CONFIGS[name]
    log(f"bias projection workload {name}: N={cfg.N} H={cfg.H} c={cfg.c}")
    inp = workloads.bias_proj_inputs(cfg)
    _check(inp, _run(inp), name)


def test_bias_proj_constant_positions_project_beta():
    """Positions whose channels are all equal have xhat = 0, so bias there is
    w . beta up to rounding; their dz is rstd = eps^-1/2 times dxhat minus its
    mean, the largest gradient in the tensor, which the full comparison covers."""
    log("bias projection constant positions")
    cfg = workloads.ProjConfig("const", N=40, H=6, c=128, seed=77)
    inp = workloads.bias_proj_inputs(cfg)
    z = inp["z"].copy()
    z[5, :, :] = z[5, :, :1]          # row 5: every channel equal to channel 0
    inp["z"] = z
    inp["z64"] = workloads.bf16_bits_to_f32(z).astype(np.float64)
    res = _run(inp)
    ref = _check(inp, res, "proj[const]")
    wb = inp["w64"] @ inp["beta64"]
    assert np.allclose(ref["bias"][:, 5, :], wb[:, None], atol=1e-12)
    assert np.allclose(res["bias"][:, 5, :], wb[:, None], rtol=1e-2, atol=1e-2 * np.abs(wb).max())
    assert np.abs(ref["dz"][5]).max() > 10 * np.abs(np.delete(ref["dz"], 5, axis=0)).max()


def test_bias_proj_backward_is_bitwise_deterministic():
    log("bias projection determinism")
    inp = workloads.bias_proj_inputs(workloads.ProjConfig("det", N=200, H=16, c=128, seed=9))
    d = _dev(inp)
    a = pba.pba_bias_proj_backward(d["z"], d["gamma"], d["beta"], d["w"], d["dbias"], EPS)
    b = pba.pba_bias_proj_backward(d["z"], d["gamma"], d["beta"], d["w"], d["dbias"], EPS)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k].view(torch.int32),
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k].view(torch.int32)), k


def test_bias_proj_outputs_stay_inside_their_buffers():
    """Ragged sizes: every output lives inside a larger buffer filled with a
    sentinel; nothing before or after the output may change."""
    log("bias projection output bounds")
    lib = pba._lib.load()
    N, H, c = 29, 5, 64                     # 841 positions: last tile holds 9
    inp = workloads.bias_proj_inputs(workloads.ProjConfig("bounds", N=N, H=H, c=c, seed=11))
    d = _dev(inp)
    pad = 4096
    sentinel_bf16 = -12345                  # int16 bit pattern
    bias_buf = torch.full((pad + H * N * N + pad,), sentinel_bf16, dtype=torch.int16, device="cuda")
    dz_buf = torch.full((pad + N * N * c + pad,), sentinel_bf16, dtype=torch.int16, device="cuda")
    f32 = {n: torch.full((pad + m + pad,), -7.0, dtype=torch.float32, device="cuda")
           for n, m in (("dgamma", c), ("dbeta", c), ("dw", H * c))}
    ws = torch.empty(lib.pba_bias_proj_backward_workspace_bytes(N, H, c, 1), dtype=torch.uint8, device="cuda")
    st = lib.pba_bias_proj_forward(N, H, c, 1, d["z"].data_ptr(), d["gamma"].data_ptr(), d["beta"].data_ptr(),
                                   d["w"].data_ptr(), EPS, bias_buf.data_ptr() + 2 * pad, None)
    assert st == 0
    st = lib.pba_bias_proj_backward(N, H, c, 1, d["z"].data_ptr(), d["gamma"].data_ptr(), d["beta"].data_ptr(),
                                    d["w"].data_ptr(), EPS, d["dbias"].data_ptr(), dz_buf.data_ptr() + 2 * pad,
                                    f32["dgamma"].data_ptr() + 4 * pad, f32["dbeta"].data_ptr() + 4 * pad,
                                    f32["dw"].data_ptr() + 4 * pad, ws.data_ptr(), ws.numel(), None)
    assert st == 0
    torch.cuda.synchronize()
    for name, buf, n in (("bias", bias_buf, H * N * N), ("dz", dz_buf, N * N * c)):
        assert bool((buf[:pad] == sentinel_bf16).all()) and bool((buf[pad + n:] == sentinel_bf16).all()), name
        assert not bool((buf[pad:pad + n] == sentinel_bf16).any()), name
    for name, n in (("dgamma", c), ("dbeta", c), ("dw", H * c)):
        buf = f32[name]
        assert bool((buf[:pad] == -7.0).all()) and bool((buf[pad + n:] == -7.0).all()), name
    res = {"bias": to_f64(bias_buf[pad:pad + H * N * N].view(torch.bfloat16).view(H, N, N)),
           "dz": to_f64(dz_buf[pad:pad + N * N * c].view(torch.bfloat16).view(N, N, c)),
           "dgamma": f32["dgamma"][pad:pad + c].cpu().numpy().astype(np.float64),
           "dbeta": f32["dbeta"][pad:pad + c].cpu().numpy().astype(np.float64),
           "dw": f32["dw"][pad:pad + H * c].view(H, c).cpu().numpy().astype(np.float64)}
    _check(inp, res, "proj[bounds]")


def test_bias_proj_feeds_attention_end_to_end():
    """z -> bias (projection) -> attention forward/backward -> dbias ->
    projection backward -> dz, all on the GPU, against the same chain in the
    fp64 oracle (no GPU value enters the oracle)."""
    log("bias projection + attention chain")
    N, H, c, B, d = 96, 4, 128, 6, 32
    pin = workloads.bias_proj_inputs(workloads.ProjConfig("chain", N=N, H=H, c=c, seed=21))
    ain = workloads.attention_inputs(workloads.AttnConfig("chain", B=B, H=H, N=N, d=d, dtype="bf16",
                                                          mask="tail:5", seed=22))
    dp = _dev(pin)
    bias = pba.pba_bias_proj_forward(dp["z"], dp["gamma"], dp["beta"], dp["w"], EPS)
    t = {n: to_dev(ain[n], "bf16") for n in ("q", "k", "v", "g", "dout")}
    km = to_dev(ain["key_mask"], "bf16")
    out, lse = pba.pba_forward(t["q"], t["k"], t["v"], t["g"], bias, km)
    ag = pba.pba_backward(t["q"], t["k"], t["v"], t["g"], bias, km, out, lse, t["dout"])
    pg = pba.pba_bias_proj_backward(dp["z"], dp["gamma"], dp["beta"], dp["w"], ag["dbias"], EPS)
    torch.cuda.synchronize()

    args = (pin["z64"], pin["gamma64"], pin["beta64"], pin["w64"])
    rbias = oracle.bias_projection_forward(*args, eps=EPS)
    O, _ = oracle.attention_forward(ain["q64"], ain["k64"], ain["v64"], ain["g64"], rbias, ain["key_mask"])
    rg = oracle.attention_backward(ain["q64"], ain["k64"], ain["v64"], ain["g64"], rbias, ain["key_mask"],
                                   ain["dout64"])
    rp = oracle.bias_projection_backward(*args, rg["dbias"], eps=EPS)
    pairs = {"bias": (to_f64(bias), rbias), "out": (to_f64(out), O)}
    pairs.update({n: (to_f64(ag[n]), rg[n]) for n in ("dq", "dv", "dbias")})
    pairs.update({n: (to_f64(pg[n]), rp[n]) for n in ("dz", "dgamma", "dbeta", "dw")})
    # every softmax row of dS sums to zero, so the attention's dbias sums to zero
    # over all positions of each head and dbeta = sum_h w[h] sum_p dbias[h, p]
    # vanishes analytically: its bar is relative to dgamma, the same kind of sum
    # over positions that does not vanish
    assert np.abs(rp["dbeta"]).max() < 1e-9 * np.abs(rp["dgamma"]).max()
    floors = {"dbeta": float(np.max(np.abs(rp["dgamma"])))}
    check_all("proj+attention", pairs, TOL["bf16"], floors)
