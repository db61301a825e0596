"""Plain fp64 CPU oracle for pair-biased gated attention and pair-weighted averaging.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and imports nothing from it; it needs NumPy only.

Every function here is the plain definition of what the method computes,
written out in float64 with NumPy matrix products as the only library
primitive.  There is no tiling, no online softmax and no fusion: the full
score matrix of one broadcast-axis chunk is materialised.  Chunking over the
broadcast axis (rows / copies / MSA rows) only bounds host memory; it does not
change any sum.

Sources, all on the AlphaFold3 open-source implementation page (molayo1419.me,
"Show HN: AlphaFold3 open-source implementation"; the same README is mirrored
on gittoolsai.com):

* section "Model Efficiency": the pair bias is projected from the pair
  representation and added after the key-query dot product; it needs a
  gradient; that gradient equals the gradient of the scaled QK^T product; and
  the forward broadcast of the bias over rows/copies becomes a reduction in the
  backward pass.  The 48 diffusion copies are treated as an extra batch axis.
* section "MSA Pair Averaging Efficiency": the MSA pair-weighted average
  replaces MSA row attention with a cheaper weighted average whose weights come
  from the pair bias only (no query-key term); the naive form materialises a
  (*, N_seq, N_res, N_res, heads, c_hidden) intermediate.
* the benchmark spec's formula: softmax(Q K^T / sqrt(d) + B_pair + mask) V,
  multiplied elementwise by sigmoid(G).

Readings where the pages are silent:
* the 1/sqrt(d) scale multiplies Q K^T only, with d the real head dimension;
* the key mask is a [N] byte vector (0 = masked, nonzero = keep) shared over
  batch, heads and queries; a masked key gets logit -inf, so its weight is 0;
* a query whose keys are all masked gets O = 0, LSE = -inf and zero gradients;
* the gate is elementwise on the normalised attention output, G has the
  shape of Q;
* bias[h, i, j] is indexed (head, query, key) and broadcast over the batch;
* the pair-weighted average has no scale and layout [S, N, H, d].

Parity: every function is pinned by the CPU tests in ``tests/test_oracle.py``
(closed forms, a reduction to a library attention routine, central finite
differences, brute force, invariants).  No function here is "parity unpinned".
"""
from __future__ import annotations

import math
import numpy as np

__all__ = [
    "sigmoid", "attention_forward", "attention_backward",
    "pwa_forward", "pwa_backward", "pwa_forward_naive",
]


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + e^-x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def _softmax_rows(logits: np.ndarray):
    """Softmax over the last axis of a logit array that may hold -inf.

    Returns (P, lse).  A row whose entries are all -inf gets P = 0 and
    lse = -inf (the fully-masked reading).
    """
    m = np.max(logits, axis=-1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(logits - m_safe)
    l = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
        lse = np.where(l > 0, m_safe + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return P, lse[..., 0]


def _logits(q, k, bias_b, keep, scale):
    """L[h, i, j] = scale * (q_i . k_j) + bias[h, i, j]; masked keys -> -inf."""
    L = np.matmul(q, np.swapaxes(k, -1, -2)) * scale + bias_b
    if keep is not None:
        L = np.where(keep[None, None, :], L, -np.inf)
    return L


def _check_attention_args(q, k, v, g, bias, key_mask):
    """Shapes: q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,dv], g [B,H,Nq,dv],
    bias [H,Nq,Nk] or [B,H,Nq,Nk], key_mask [Nk].  Every workload has Nq = Nk
    and dv = d; the general form lets a test take a subset of query rows."""
    B, H, Nq, d = q.shape
    if k.ndim != 4 or k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError(f"k has shape {k.shape}, expected {(B, H)} + (Nk, {d})")
    Nk = k.shape[2]
    if v.ndim != 4 or v.shape[:3] != (B, H, Nk):
        raise ValueError(f"v has shape {v.shape}, expected {(B, H, Nk)} + (dv,)")
    if g.shape != (B, H, Nq, v.shape[3]):
        raise ValueError(f"g has shape {g.shape}, expected {(B, H, Nq, v.shape[3])}")
    if bias.shape not in ((H, Nq, Nk), (B, H, Nq, Nk)):
        raise ValueError(f"bias has shape {bias.shape}, expected {(H, Nq, Nk)} or {(B, H, Nq, Nk)}")
    keep = None
    if key_mask is not None:
        keep = np.asarray(key_mask).reshape(Nk) != 0
    return B, H, Nq, d, keep


def attention_forward(q, k, v, g, bias, key_mask=None, scale=None, chunk=32):
    """Forward pass of pair-biased gated attention, per (batch row b, head h).

    O[b,h,i,:] = sigmoid(G[b,h,i,:]) * sum_j P[b,h,i,j] V[b,h,j,:], with
    P = softmax_j(scale * Q K^T + bias[h] + mask).  Returns (O, LSE) where
    LSE[b,h,i] = log sum_j exp(logit[b,h,i,j]) (natural log).

    q, k: [B, H, N, d]; v, g: [B, H, N, dv] (dv = d in every workload);
    bias: [H, N, N] shared over B, or [B, H, N, N].  (Query and key counts
    may differ; see _check_attention_args.)
    """
    q, k, v, g, bias = (np.asarray(t, dtype=np.float64) for t in (q, k, v, g, bias))
    B, H, N, d, keep = _check_attention_args(q, k, v, g, bias, key_mask)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.empty(g.shape)
    LSE = np.empty((B, H, N))
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        bias_b = bias if bias.ndim == 3 else bias[b0:b1]
        L = _logits(q[b0:b1], k[b0:b1], bias_b, keep, scale)
        P, lse = _softmax_rows(L)
        A = np.matmul(P, v[b0:b1])
        O[b0:b1] = sigmoid(g[b0:b1]) * A
        LSE[b0:b1] = lse
    return O, LSE


def attention_backward(q, k, v, g, bias, key_mask, dout, scale=None, chunk=32):
    """Gradients of L = sum(O * dout) for pair-biased gated attention.

    Written from the plain chain rule (no softmax shortcut through O):
      A = P V,  O = s * A with s = sigmoid(G)
      dA = dout * s,  dG = dout * A * s * (1 - s)
      dV = P^T dA,  dP = dA V^T
      dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)          (softmax Jacobian)
      dQ = scale * dS K,  dK = scale * dS^T Q
      dBias = dS, reduced over the batch axis when the bias is broadcast
    The last line is the "Model Efficiency" statement: the bias gradient is the
    gradient of the scaled QK^T product, and the broadcast becomes a reduction.

    Returns a dict with dq, dk, dv, dg ([B,H,N,d]) and dbias (bias's shape).
    """
    q, k, v, g, bias, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, g, bias, dout))
    B, H, N, d, keep = _check_attention_args(q, k, v, g, bias, key_mask)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dg = np.empty_like(g)
    dbias = np.zeros_like(bias)
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        sl = slice(b0, b1)
        bias_b = bias if bias.ndim == 3 else bias[sl]
        L = _logits(q[sl], k[sl], bias_b, keep, scale)
        P, _ = _softmax_rows(L)
        A = np.matmul(P, v[sl])
        s = sigmoid(g[sl])
        dA = dout[sl] * s
        dg[sl] = dout[sl] * A * s * (1.0 - s)
        dv[sl] = np.matmul(np.swapaxes(P, -1, -2), dA)
        dP = np.matmul(dA, np.swapaxes(v[sl], -1, -2))
        dS = P * (dP - np.sum(P * dP, axis=-1, keepdims=True))
        dq[sl] = np.matmul(dS, k[sl]) * scale
        dk[sl] = np.matmul(np.swapaxes(dS, -1, -2), q[sl]) * scale
        if bias.ndim == 3:
            dbias += np.sum(dS, axis=0)
        else:
            dbias[sl] = dS
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dbias": dbias}


def _check_pwa_args(b, v, g, key_mask):
    """Shapes: b [H,Nq,Nk], v [S,Nk,H,d], g [S,Nq,H,d], key_mask [Nk]
    (Nq = Nk in every workload; a test may take a subset of rows i)."""
    S, Nk, H, d = v.shape
    if b.ndim != 3 or b.shape[0] != H or b.shape[2] != Nk:
        raise ValueError(f"b has shape {b.shape}, expected {(H,)} + (Nq, {Nk})")
    Nq = b.shape[1]
    if g.shape != (S, Nq, H, d):
        raise ValueError(f"g has shape {g.shape}, expected {(S, Nq, H, d)}")
    keep = None
    if key_mask is not None:
        keep = np.asarray(key_mask).reshape(Nk) != 0
    return S, Nk, H, d, keep


def _pwa_weights(b, keep):
    L = b if keep is None else np.where(keep[None, None, :], b, -np.inf)
    return _softmax_rows(L)


def pwa_forward(b, v, g, key_mask=None, chunk=128):
    """MSA pair-weighted averaging ("MSA Pair Averaging Efficiency" section).

    w[h,i,j] = softmax_j(b[h,i,j] + mask);
    O[s,i,h,:] = sigmoid(G[s,i,h,:]) * sum_j w[h,i,j] V[s,j,h,:].
    b: [H, N, N]; v, g: [S, N, H, d].  Returns (O, lse_w) with lse_w [H, N].
    (Row and token counts may differ; see _check_pwa_args.)
    """
    b, v, g = (np.asarray(t, dtype=np.float64) for t in (b, v, g))
    S, Nk, H, d, keep = _check_pwa_args(b, v, g, key_mask)
    Nq = b.shape[1]
    w, lse = _pwa_weights(b, keep)
    O = np.empty(g.shape)
    for s0 in range(0, S, chunk):
        s1 = min(S, s0 + chunk)
        n = s1 - s0
        for h in range(H):
            # [Nq, Nk] @ [Nk, (s, c)] per head, with the MSA rows as extra columns
            vh = np.transpose(v[s0:s1, :, h, :], (1, 0, 2)).reshape(Nk, n * d)
            Ah = (w[h] @ vh).reshape(Nq, n, d).transpose(1, 0, 2)
            O[s0:s1, :, h, :] = sigmoid(g[s0:s1, :, h, :]) * Ah
    return O, lse


def pwa_backward(b, v, g, key_mask, dout, chunk=128):
    """Gradients of sum(O * dout) for the pair-weighted average.

      A = w V (per head, per MSA row),  O = s * A,  s = sigmoid(G)
      dA = dout * s,  dG = dout * A * s * (1 - s)
      dV[s,j,h,:] = sum_i w[h,i,j] dA[s,i,h,:]
      dw[h,i,j]   = sum_{s,c} dA[s,i,h,c] V[s,j,h,c]   (broadcast over s -> reduction)
      db = w * (dw - sum_j w * dw)                      (softmax Jacobian)
    Returns a dict with dv, dg ([S,N,H,d]) and db ([H,N,N]).  With a subset of
    rows i, dv holds only those rows' contributions.
    """
    b, v, g, dout = (np.asarray(t, dtype=np.float64) for t in (b, v, g, dout))
    S, Nk, H, d, keep = _check_pwa_args(b, v, g, key_mask)
    Nq = b.shape[1]
    w, _ = _pwa_weights(b, keep)
    dv = np.empty_like(v)
    dg = np.empty_like(g)
    dw = np.zeros((H, Nq, Nk))
    for s0 in range(0, S, chunk):
        s1 = min(S, s0 + chunk)
        n = s1 - s0
        for h in range(H):
            vh = np.transpose(v[s0:s1, :, h, :], (1, 0, 2)).reshape(Nk, n * d)
            Ah = (w[h] @ vh).reshape(Nq, n, d).transpose(1, 0, 2)
            sh = sigmoid(g[s0:s1, :, h, :])
            dAh = dout[s0:s1, :, h, :] * sh
            dg[s0:s1, :, h, :] = dout[s0:s1, :, h, :] * Ah * sh * (1.0 - sh)
            dAh_m = np.transpose(dAh, (1, 0, 2)).reshape(Nq, n * d)
            dv[s0:s1, :, h, :] = (w[h].T @ dAh_m).reshape(Nk, n, d).transpose(1, 0, 2)
            dw[h] += dAh_m @ vh.T
    db = w * (dw - np.sum(w * dw, axis=-1, keepdims=True))
    return {"dv": dv, "dg": dg, "db": db}


def pwa_forward_naive(b, v, g, key_mask=None):
    """The naive pair-weighted average that materialises the 6-D intermediate.

    The "MSA Pair Averaging Efficiency" section describes the naive
    implementation as allocating a (*, N_seq, N_res, N_res, heads, c_hidden)
    tensor; this builds exactly that product w[h,i,j] * V[s,j,h,c] indexed
    [s, i, j, h, c] and sums it over j.  Tiny inputs only.
    """
    b, v, g = (np.asarray(t, dtype=np.float64) for t in (b, v, g))
    S, N, H, d, keep = _check_pwa_args(b, v, g, key_mask)
    w, _ = _pwa_weights(b, keep)
    inter = np.transpose(w, (1, 2, 0))[None, :, :, :, None] * v[:, None, :, :, :]
    return sigmoid(g) * inter.sum(axis=2)
