"""CPU pins of the fp64 pair-bias projection oracle (bias = Linear(LayerNorm(z))).

The oracle writes out LayerNorm, the affine step, the projection and the chain
rule by hand; these tests hold it to things other than itself: PyTorch's own
layer_norm + linear with autograd in fp64 (a library routine), central finite
differences, closed forms and invariants.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _case(N=5, c=16, H=3, seed=0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((N, N, c)) * 1.5 + 0.3
    gamma = 1.0 + 0.2 * rng.standard_normal(c)
    beta = 0.1 * rng.standard_normal(c)
    w = rng.standard_normal((H, c)) / math.sqrt(c)
    dbias = rng.standard_normal((H, N, N))
    return z, gamma, beta, w, dbias


def test_matches_library_layer_norm_and_linear():
    z, gamma, beta, w, dbias = _case()
    tz = torch.tensor(z, requires_grad=True)
    tg = torch.tensor(gamma, requires_grad=True)
    tb = torch.tensor(beta, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    y = torch.nn.functional.layer_norm(tz, (z.shape[-1],), tg, tb, eps=oracle.BIAS_PROJ_EPS)
    out = torch.nn.functional.linear(y, tw).permute(2, 0, 1)
    out.backward(torch.tensor(dbias))
    ref = out.detach().numpy()
    got = oracle.bias_projection_forward(z, gamma, beta, w)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    gr = oracle.bias_projection_backward(z, gamma, beta, w, dbias)
    for name, t in (("dz", tz), ("dgamma", tg), ("dbeta", tb), ("dw", tw)):
        assert np.allclose(gr[name], t.grad.numpy(), rtol=1e-10, atol=1e-12), name


def test_gradients_match_central_differences():
    z, gamma, beta, w, dbias = _case(N=3, c=8, H=2, seed=1)
    gr = oracle.bias_projection_backward(z, gamma, beta, w, dbias)

    def loss(z_, g_, b_, w_):
        return float(np.sum(oracle.bias_projection_forward(z_, g_, b_, w_) * dbias))

    h = 1e-6
    args = [z, gamma, beta, w]
    for idx, name in enumerate(("dz", "dgamma", "dbeta", "dw")):
        base = args[idx]
        num = np.zeros_like(base)
        for pos in np.ndindex(base.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[idx][pos] += h
            minus[idx][pos] -= h
            num[pos] = (loss(*plus) - loss(*minus)) / (2 * h)
        err = np.max(np.abs(num - gr[name])) / max(1e-12, np.max(np.abs(gr[name])))
        assert err < 1e-7, (name, err)


def test_constant_channels_project_beta():
    # every channel equal: xhat = 0, so y = beta and bias = w . beta at every position
    N, c, H = 4, 8, 3
    rng = np.random.default_rng(2)
    z = np.repeat(rng.standard_normal((N, N, 1)), c, axis=-1)
    gamma = rng.standard_normal(c)
    beta = rng.standard_normal(c)
    w = rng.standard_normal((H, c))
    got = oracle.bias_projection_forward(z, gamma, beta, w)
    assert np.allclose(got, (w @ beta)[:, None, None] * np.ones((1, N, N)), atol=1e-12)


def test_two_channel_closed_form():
    # c = 2: the normalised pair is +-a with a = |z0 - z1| / 2 / sqrt(((z0 - z1)/2)^2 + eps)
    z = np.array([[[3.0, -1.0]]])
    gamma = np.array([1.0, 1.0])
    beta = np.array([0.0, 0.0])
    w = np.array([[1.0, 0.0], [0.0, 1.0]])
    eps = oracle.BIAS_PROJ_EPS
    half = 2.0
    a = half / math.sqrt(half * half + eps)
    got = oracle.bias_projection_forward(z, gamma, beta, w)
    assert np.allclose(got[:, 0, 0], [a, -a], atol=1e-14)


def test_identity_projection_gives_layer_norm_channels():
    # gamma = 1, beta = 0, w = unit rows: bias[h] is LayerNorm channel h, checked by
    # a plain loop over positions and channels
    N, c = 3, 6
    rng = np.random.default_rng(3)
    z = rng.standard_normal((N, N, c))
    w = np.eye(c)[:4]
    got = oracle.bias_projection_forward(z, np.ones(c), np.zeros(c), w)
    eps = oracle.BIAS_PROJ_EPS
    for i in range(N):
        for j in range(N):
            vals = [float(x) for x in z[i, j]]
            m = sum(vals) / c
            v = sum((x - m) ** 2 for x in vals) / c
            for h in range(4):
                assert abs(got[h, i, j] - (vals[h] - m) / math.sqrt(v + eps)) < 1e-12


def test_invariants():
    z, gamma, beta, w, dbias = _case(seed=4)
    gr = oracle.bias_projection_backward(z, gamma, beta, w, dbias)
    # LayerNorm removes the mean: its input gradient sums to zero over channels
    assert np.allclose(gr["dz"].sum(axis=-1), 0.0, atol=1e-12)
    # shifting every channel of z by a constant changes nothing
    shift = 7.5
    assert np.allclose(oracle.bias_projection_forward(z + shift, gamma, beta, w),
                       oracle.bias_projection_forward(z, gamma, beta, w), atol=1e-10)
    g2 = oracle.bias_projection_backward(z + shift, gamma, beta, w, dbias)
    assert np.allclose(g2["dz"], gr["dz"], atol=1e-9)
    # the projection is linear in w and beta enters every position once
    H = w.shape[0]
    assert np.allclose(gr["dbeta"], w.T @ dbias.reshape(H, -1).sum(axis=1), atol=1e-10)
    # with w = 0 no gradient reaches y, so dz vanishes while dw = dbias (x) y does not
    z0 = oracle.bias_projection_backward(z, gamma, beta, np.zeros_like(w), dbias)
    assert np.all(z0["dz"] == 0) and np.all(z0["dw"] != 0)
