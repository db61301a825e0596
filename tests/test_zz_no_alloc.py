"""The allocation-free backward entry point (pba_backward_noalloc), called
through the C ABI, against pba_backward with a caller-owned workspace.

Both run the same kernels with the same plan, so the outputs must agree
bit for bit.  Two calls in a row, the second with a smaller input, check
that the shared static scratch area carries nothing from one call into the
next; an oversized call must be refused before anything is enqueued.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import pair_biased_attention_amd._lib as L
    return L.load()  # fails loudly if the library is missing


def _inputs(B, H, N, d, dtype, mask, seed):
    cfg = workloads.AttnConfig("noalloc", B=B, H=H, N=N, d=d, dtype=dtype, mask=mask, seed=seed)
    inp = workloads.attention_inputs(cfg, with_f64=False)
    dev = {n: to_dev(inp[n], dtype) for n in ("q", "k", "v", "g", "bias", "dout")}
    dev["key_mask"] = None if inp["key_mask"] is None else to_dev(inp["key_mask"], dtype)
    return dev


def _grads(q, bias):
    g = {n: torch.empty_like(q) for n in ("dq", "dk", "dv", "dg")}
    g["dbias"] = torch.empty_like(bias)
    return g


def _both(lib, dev, dt):
    import pair_biased_attention_amd as pba
    q = dev["q"]
    B, H, N, d = q.shape
    out, lse = pba.pba_forward(q, dev["k"], dev["v"], dev["g"], dev["bias"], dev["key_mask"])
    p = lambda t: None if t is None else t.data_ptr()
    args = (B, H, N, d, dt, p(q), p(dev["k"]), p(dev["v"]), p(dev["g"]), p(dev["bias"]), p(dev["key_mask"]),
            p(out), p(lse), p(dev["dout"]))
    ref = _grads(q, dev["bias"])
    wsb = lib.pba_backward_workspace_bytes(B, H, N, d, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    st = lib.pba_backward(*args, *(p(ref[n]) for n in ("dq", "dk", "dv", "dg", "dbias")), p(ws), wsb, None)
    assert st == 0, st
    got = _grads(q, dev["bias"])
    # fill the outputs so that a missing write shows
    for t in got.values():
        t.fill_(-7.0)
    st = lib.pba_backward_noalloc(*args, *(p(got[n]) for n in ("dq", "dk", "dv", "dg", "dbias")), None)
    assert st == 0, lib.pba_status_string(st)
    torch.cuda.synchronize()
    for n in ref:
        a = ref[n].view(torch.int16 if ref[n].dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        b = got[n].view(torch.int16 if got[n].dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        assert np.array_equal(a, b), f"{n}: pba_backward_noalloc differs from pba_backward"


def test_noalloc_matches_workspace_backward_twice(lib):
    log("no-alloc backward: B=96 H=4 N=384 d=32 bf16 (tail mask), then B=3 H=2 N=100 d=24 (random mask)")
    _both(lib, _inputs(96, 4, 384, 32, "bf16", "tail:19", 61), 1)
    log("no-alloc backward: second, smaller call")
    _both(lib, _inputs(3, 2, 100, 24, "bf16", "random:5", 62), 1)
    log("no-alloc backward: fp32, N=40")
    _both(lib, _inputs(4, 2, 40, 32, "f32", "random:3", 63), 0)


def test_noalloc_refuses_oversized_call(lib):
    import pair_biased_attention_amd._lib as L
    B, H, N, d = 1024, 8, 768, 32
    assert lib.pba_backward_workspace_bytes(B, H, N, d, 1) > L.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.uint8, device="cuda")  # never dereferenced: refused first
    p = x.data_ptr()
    st = lib.pba_backward_noalloc(B, H, N, d, 1, *([p] * 5), None, *([p] * 8), None)
    assert st == 7, lib.pba_status_string(st)
