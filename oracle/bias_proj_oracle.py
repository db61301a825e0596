"""Plain fp64 CPU oracle for the pair-bias projection bias = Linear(LayerNorm(z)).

TEST INFRASTRUCTURE ONLY, under the same rules as ``pba_oracle``: only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import it; it shares no code with the HIP library and needs NumPy only.

What is computed (AlphaFold3 open-source implementation page, molayo1419.me,
section "Model Efficiency": every attention projects its pair bias from the
pairwise representation, and that bias needs a gradient; the Protenix page
names LayerNorm as a kernel worth a custom implementation):

    for every pair position (i, j) of z [N, N, c]:
        mean  = (1/c) sum_k z[i,j,k]
        var   = (1/c) sum_k (z[i,j,k] - mean)^2            (biased variance)
        xhat  = (z[i,j,:] - mean) / sqrt(var + eps)
        y     = gamma * xhat + beta                          (affine LayerNorm)
        bias[h, i, j] = sum_k w[h, k] * y[k]                 (linear, no offset)

Readings where the pages are silent: the projection is
LayerNorm followed by a linear map without an offset term, the LayerNorm is
affine with eps = 1e-5 and the biased variance, the output is laid out
[H, N, N] (head, query, key) as the attention consumes it.

The backward takes dbias [H, N, N] (the attention's dBias) and returns dz,
dgamma, dbeta and dw by the chain rule written out step by step: the
gradient reaching y, the affine parameters' sums over all positions, and the
LayerNorm's own Jacobian applied to dxhat.

Parity: every function is pinned by ``tests/test_bias_proj_oracle.py``
(central finite differences, the reduction to a library LayerNorm + linear in
fp64, closed forms, invariants).  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = ["bias_projection_forward", "bias_projection_backward", "BIAS_PROJ_EPS"]

BIAS_PROJ_EPS = 1e-5


def _normalise(z, eps):
    z = np.asarray(z, dtype=np.float64)
    mean = z.mean(axis=-1, keepdims=True)
    var = ((z - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    return (z - mean) * rstd, rstd


def bias_projection_forward(z, gamma, beta, w, eps=BIAS_PROJ_EPS):
    """bias [H, N, N] = w . (gamma * LayerNorm(z) + beta) at every pair position."""
    z = np.asarray(z, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N1, N2, c = z.shape
    assert w.shape[1] == c and gamma.shape == (c,) and beta.shape == (c,)
    xhat, _ = _normalise(z, eps)
    y = xhat * gamma + beta                                   # [N, N, c]
    bias = y.reshape(N1 * N2, c) @ w.T                        # [N*N, H]
    return np.ascontiguousarray(bias.T.reshape(w.shape[0], N1, N2))


def bias_projection_backward(z, gamma, beta, w, dbias, eps=BIAS_PROJ_EPS):
    """Gradients of bias_projection_forward given dbias [H, N, N]:
    returns dict(dz [N,N,c], dgamma [c], dbeta [c], dw [H,c])."""
    z = np.asarray(z, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dbias = np.asarray(dbias, dtype=np.float64)
    N1, N2, c = z.shape
    H = w.shape[0]
    xhat, rstd = _normalise(z, eps)
    y = xhat * gamma + beta
    db = dbias.reshape(H, N1 * N2).T                          # [N*N, H]: gradient at each position
    dy = (db @ w).reshape(N1, N2, c)                          # d bias / d y = w
    dw = db.T @ y.reshape(N1 * N2, c)                         # [H, c]
    dgamma = (dy * xhat).sum(axis=(0, 1))
    dbeta = dy.sum(axis=(0, 1))
    dxhat = dy * gamma
    # Jacobian of xhat = (z - mean) * rstd with respect to z, per position
    dz = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True)
                 - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    return {"dz": dz, "dgamma": dgamma, "dbeta": dbeta, "dw": dw}
