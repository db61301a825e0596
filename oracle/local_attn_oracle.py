"""Plain fp64 CPU oracle for windowed (sequence-local) pair-biased gated attention.

TEST INFRASTRUCTURE ONLY, under the same rules as ``pba_oracle``: only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import it; it shares no code with the HIP library and needs NumPy only.

What is computed.  The AlphaFold3 open-source implementation page
(molayo1419.me), section "Model Efficiency", says that for the
AtomAttentionEncoder and AtomAttentionDecoder the authors tried an
implementation whose memory grows linearly rather than quadratically with the
number of atoms, next to the plain reuse of the AttentionPairBias kernel.
Linear memory means each query attends a fixed-size window of keys and the
pair bias exists only inside the windows:

    query block q   = atoms 32q .. 32q + 31                      (WQ = 32)
    its key window  = atoms 32q - 48 .. 32q + 79, slots s = 0..127 (WK = 128)
    L[b,h,i,s] = Q[b,h,i] . K[b,h,32q - 48 + s] / sqrt(d) + bias[h, q, i - 32q, s]
                 (-inf for slots outside [0, N) and for masked keys)
    P = softmax_s(L),  A = P V,  O = sigmoid(G) * A,  lse = log sum_s exp(L)

and the backward returns dQ, dK, dV, dG and dbias = sum_b dS (the bias is
broadcast over the batch axis, as in the dense kernel).

Readings where the pages are silent: the window shape (32 queries, 128 keys,
centred on the query block), the local bias layout [H, ceil(N/32), 32, 128]
indexed (head, query block, query in block, slot), and that query rows past N
in the last block produce nothing and get a zero bias gradient.  Everything
else (scale, key mask, gate, natural-log lse, fully masked rows) follows the
dense oracle's readings.

Parity: pinned by ``tests/test_local_attn_oracle.py`` (a library attention
routine with a dense mask and autograd, central finite differences, the
reduction to dense attention when every window covers every key, locality and
invariants).  No function here is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["LOCAL_WQ", "LOCAL_WK", "LOCAL_WOFF", "local_window_keys",
           "local_attention_forward", "local_attention_backward"]

LOCAL_WQ = 32    # queries per block
LOCAL_WK = 128   # keys per window
LOCAL_WOFF = 48  # the window starts this many atoms before its query block


def local_window_keys(qb: int) -> np.ndarray:
    """Atom index of every slot of query block qb's window (may lie outside [0, N))."""
    return LOCAL_WQ * qb - LOCAL_WOFF + np.arange(LOCAL_WK)


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _blocks(N, key_mask):
    """Per query block: (query rows, usable slot flags, their key indices)."""
    keep = np.ones(N, dtype=bool) if key_mask is None else np.asarray(key_mask) != 0
    out = []
    for qb in range(-(-N // LOCAL_WQ)):
        rows = np.arange(LOCAL_WQ * qb, min(LOCAL_WQ * qb + LOCAL_WQ, N))
        keys = local_window_keys(qb)
        usable = (keys >= 0) & (keys < N)
        usable[usable] = keep[keys[usable]]
        out.append((qb, rows, usable, keys[usable]))
    return out


def _check(q, k, v, g, bias):
    B, H, N, d = q.shape
    assert k.shape == v.shape == g.shape == q.shape
    assert bias.shape == (H, -(-N // LOCAL_WQ), LOCAL_WQ, LOCAL_WK), bias.shape
    return B, H, N, d


def local_attention_forward(q, k, v, g, bias, key_mask=None, scale=None):
    """O [B,H,N,d] and lse [B,H,N] (natural log; -inf for a row without usable keys)."""
    q, k, v, g, bias = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, bias))
    B, H, N, d = _check(q, k, v, g, bias)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.zeros_like(q)
    lse = np.full((B, H, N), -np.inf)
    for qb, rows, usable, kv in _blocks(N, key_mask):
        if kv.size == 0:
            continue
        logits = np.matmul(q[:, :, rows], np.swapaxes(k[:, :, kv], -1, -2)) * scale
        logits = logits + bias[None, :, qb, :rows.size][..., usable]
        m = logits.max(axis=-1, keepdims=True)
        e = np.exp(logits - m)
        l = e.sum(axis=-1, keepdims=True)
        p = e / l
        a = np.matmul(p, v[:, :, kv])
        out[:, :, rows] = _sigmoid(g[:, :, rows]) * a
        lse[:, :, rows] = (m + np.log(l))[..., 0]
    return out, lse


def local_attention_backward(q, k, v, g, bias, key_mask, dout, scale=None):
    """dict(dq, dk, dv, dg [B,H,N,d]; dbias [H, nqb, 32, 128] summed over B)."""
    q, k, v, g, bias, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, bias, dout))
    B, H, N, d = _check(q, k, v, g, bias)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq, dk, dv, dg = (np.zeros_like(q) for _ in range(4))
    dbias = np.zeros_like(bias)
    for qb, rows, usable, kv in _blocks(N, key_mask):
        if kv.size == 0:
            continue
        qs, ks, vs = q[:, :, rows], k[:, :, kv], v[:, :, kv]
        logits = np.matmul(qs, np.swapaxes(ks, -1, -2)) * scale + bias[None, :, qb, :rows.size][..., usable]
        e = np.exp(logits - logits.max(axis=-1, keepdims=True))
        p = e / e.sum(axis=-1, keepdims=True)
        a = np.matmul(p, vs)
        sg = _sigmoid(g[:, :, rows])
        da = dout[:, :, rows] * sg
        dg[:, :, rows] = dout[:, :, rows] * a * sg * (1.0 - sg)
        dv[:, :, kv] += np.matmul(np.swapaxes(p, -1, -2), da)
        dp = np.matmul(da, np.swapaxes(vs, -1, -2))
        ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))   # softmax Jacobian per row
        dq[:, :, rows] = np.matmul(ds, ks) * scale
        dk[:, :, kv] += np.matmul(np.swapaxes(ds, -1, -2), qs) * scale
        blk = np.zeros((H, rows.size, LOCAL_WK))
        blk[..., usable] = ds.sum(axis=0)
        dbias[:, qb, :rows.size] = blk
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dbias": dbias}
