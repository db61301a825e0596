"""CPU pins of the fp64 windowed-attention oracle (``oracle/local_attn_oracle.py``).

The oracle is held to things other than itself: PyTorch's scaled-dot-product
attention (a library routine) with the window written as a dense additive
mask, in fp64 with autograd for every gradient; the dense attention oracle
(itself pinned in test_oracle.py) where every window covers every key; central
finite differences; locality; and invariants of the softmax Jacobian.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

WQ, WK, OFF = oracle.LOCAL_WQ, oracle.LOCAL_WK, oracle.LOCAL_WOFF


def _case(B=2, H=2, N=70, d=8, seed=0, masked=()):
    rng = np.random.default_rng(seed)
    nqb = -(-N // WQ)
    q, k, v, g, dout = (rng.standard_normal((B, H, N, d)) for _ in range(5))
    bias = rng.standard_normal((H, nqb, WQ, WK))
    keep = None
    if masked:
        keep = np.ones(N, dtype=np.uint8)
        keep[list(masked)] = 0
    return q, k, v, g, bias, keep, dout


def _dense_bias(bias, N, keep):
    """[H, N, N] additive bias: the local bias inside each window, -inf elsewhere."""
    H = bias.shape[0]
    dense = np.full((H, N, N), -np.inf)
    for i in range(N):
        qb = i // WQ
        for s in range(WK):
            j = WQ * qb - OFF + s
            if 0 <= j < N and (keep is None or keep[j]):
                dense[:, i, j] = bias[:, qb, i - WQ * qb, s]
    return dense


def test_matches_library_attention_with_a_dense_window_mask():
    q, k, v, g, bias, keep, dout = _case(N=100, masked=(3, 57, 99))
    B, H, N, d = q.shape
    dense = _dense_bias(bias, N, keep)
    t = {n: torch.tensor(x, requires_grad=True) for n, x in (("q", q), ("k", k), ("v", v), ("g", g))}
    tm = torch.tensor(dense[None], requires_grad=True)
    a = torch.nn.functional.scaled_dot_product_attention(t["q"], t["k"], t["v"], attn_mask=tm,
                                                         scale=1.0 / math.sqrt(d))
    o = torch.sigmoid(t["g"]) * a
    o.backward(torch.tensor(dout))
    out, lse = oracle.local_attention_forward(q, k, v, g, bias, keep)
    assert np.allclose(out, o.detach().numpy(), rtol=1e-12, atol=1e-12)
    gr = oracle.local_attention_backward(q, k, v, g, bias, keep, dout)
    for n in ("q", "k", "v", "g"):
        assert np.allclose(gr["d" + n], t[n].grad.numpy(), rtol=1e-10, atol=1e-12), n
    dm = tm.grad.numpy()[0]
    for i in range(N):
        qb = i // WQ
        for s in range(WK):
            j = WQ * qb - OFF + s
            want = dm[:, i, j] if (0 <= j < N and keep[j]) else 0.0
            assert np.allclose(gr["dbias"][:, qb, i - WQ * qb, s], want, atol=1e-12)
    # lse from the library's logits
    logits = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(d) + dense[None]
    m = logits.max(-1)
    assert np.allclose(lse, m + np.log(np.exp(logits - m[..., None]).sum(-1)), atol=1e-12)


def test_reduces_to_dense_attention_when_windows_cover_every_key():
    # N <= 64: the windows of blocks 0 and 1 span atoms -48..79 and -16..111
    q, k, v, g, bias, keep, dout = _case(N=60, d=4, seed=1, masked=(7,))
    dense = _dense_bias(bias, 60, keep)
    assert np.isfinite(dense[:, :, [j for j in range(60) if j != 7]]).all()
    dense[~np.isfinite(dense)] = 0.0  # masked key: the key mask does the masking now
    O, L = oracle.attention_forward(q, k, v, g, dense, keep)
    out, lse = oracle.local_attention_forward(q, k, v, g, bias, keep)
    assert np.allclose(out, O, atol=1e-12) and np.allclose(lse, L, atol=1e-12)
    gd = oracle.attention_backward(q, k, v, g, dense, keep, dout)
    gl = oracle.local_attention_backward(q, k, v, g, bias, keep, dout)
    for n in ("dq", "dk", "dv", "dg"):
        assert np.allclose(gl[n], gd[n], atol=1e-12), n


def test_gradients_match_central_differences():
    q, k, v, g, bias, keep, dout = _case(B=1, H=1, N=70, d=3, seed=2, masked=(40,))
    gr = oracle.local_attention_backward(q, k, v, g, bias, keep, dout)

    def loss(q_, k_, v_, g_, b_):
        return float(np.sum(oracle.local_attention_forward(q_, k_, v_, g_, b_, keep)[0] * dout))

    rng = np.random.default_rng(3)
    args = [q, k, v, g, bias]
    h = 1e-6
    for idx, name in enumerate(("dq", "dk", "dv", "dg", "dbias")):
        base = args[idx]
        for _ in range(25):
            pos = tuple(int(rng.integers(s)) for s in base.shape)
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[idx][pos] += h
            minus[idx][pos] -= h
            num = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(num - gr[name][pos]) <= 1e-6 * max(1.0, abs(num)), (name, pos, num, gr[name][pos])


def test_locality_and_invariants():
    q, k, v, g, bias, keep, dout = _case(N=150, seed=4, masked=(10, 149))
    out, lse = oracle.local_attention_forward(q, k, v, g, bias, keep)
    # block 0 (atoms 0..31) sees keys -48..79 only: changing K, V beyond 79 leaves it alone
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 80:] += 5.0
    v2[:, :, 80:] -= 3.0
    out2, _ = oracle.local_attention_forward(q, k2, v2, g, bias, keep)
    assert np.array_equal(out2[:, :, :32], out[:, :, :32])
    assert not np.allclose(out2[:, :, 32:], out[:, :, 32:])
    gr = oracle.local_attention_backward(q, k, v, g, bias, keep, dout)
    # softmax Jacobian: every row of dS sums to zero, so does each bias-gradient row
    assert np.allclose(gr["dbias"].sum(-1), 0.0, atol=1e-12)
    # masked keys get no gradient; slots outside [0, N) and padding rows none either
    assert np.all(gr["dk"][:, :, [10, 149]] == 0) and np.all(gr["dv"][:, :, [10, 149]] == 0)
    assert np.all(gr["dbias"][:, 0, :, :OFF] == 0)              # atoms -48..-1
    nqb = bias.shape[1]
    assert np.all(gr["dbias"][:, nqb - 1, 150 - WQ * (nqb - 1):] == 0)   # rows 150..159 do not exist
    # a window whose keys are all masked: O = 0, lse = -inf, zero gradients
    keep_all = np.zeros(150, dtype=np.uint8)
    keep_all[100:] = 1          # block 0's window (keys -48..79) has no usable key
    o3, l3 = oracle.local_attention_forward(q, k, v, g, bias, keep_all)
    assert np.all(o3[:, :, :32] == 0) and np.all(np.isneginf(l3[:, :, :32]))
    g3 = oracle.local_attention_backward(q, k, v, g, bias, keep_all, dout)
    assert np.all(g3["dq"][:, :, :32] == 0) and np.all(g3["dbias"][:, 0] == 0)
