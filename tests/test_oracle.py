"""Pins for the fp64 oracle: checks against facts that do not come from the oracle.

Each test pins a part of the oracle to something independent of it: a closed
form, a library routine the oracle never calls, central finite differences,
brute force with pure-Python loops, or an invariant the mathematics fixes.
The cases are chosen so that a dropped term, a wrong sign or index or a
transposed operand in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
import workloads

RNG = np.random.default_rng(7)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def _tiny(B=2, H=2, N=5, d=3, masked=(3,), rng=None):
    rng = rng or np.random.default_rng(11)
    q, k, v, g, dout = (rng.standard_normal((B, H, N, d)) for _ in range(5))
    bias = rng.standard_normal((H, N, N))
    keep = np.ones(N, np.uint8)
    for j in masked:
        keep[j] = 0
    return q, k, v, g, bias, keep, dout


def _probs(q, k, bias, keep):
    """Extract P from the forward: V = identity over keys, G = 40 (sigmoid == 1)."""
    B, H, N, d = q.shape
    eye = np.broadcast_to(np.eye(N), (B, H, N, N)).copy()
    big = np.full((B, H, N, N), 40.0)
    P, _ = oracle.attention_forward(q, k, eye, big, bias, keep, scale=1.0 / math.sqrt(d))
    return P


# ---------------------------------------------------------------- softmax pins

def test_sigmoid_forty_is_one():
    # the "G large" reading: sigmoid(40) rounds to exactly 1.0 in fp64
    assert oracle.sigmoid(np.array([40.0]))[0] == 1.0
    assert abs(oracle.sigmoid(np.array([0.0]))[0] - 0.5) == 0.0
    x = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(oracle.sigmoid(x) + oracle.sigmoid(-x), 1.0, rtol=0, atol=1e-15)


def test_probability_rows_sum_to_one_and_mask_is_exact_zero():
    q, k, v, g, bias, keep, _ = _tiny(B=3, H=2, N=7, d=4, masked=(1, 5))
    P = _probs(q, k, bias, keep)
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert np.all(P[..., keep == 0] == 0.0)
    assert np.all(P[..., keep != 0] > 0)


def test_brute_force_loops_match():
    """Pure-Python triple loops with math.fsum against the vectorised oracle."""
    q, k, v, g, bias, keep, _ = _tiny(B=2, H=2, N=4, d=3, masked=(2,))
    O, LSE = oracle.attention_forward(q, k, v, g, bias, keep)
    B, H, N, d = q.shape
    sc = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                logits = []
                for j in range(N):
                    if not keep[j]:
                        continue
                    dot = math.fsum(q[b, h, i, c] * k[b, h, j, c] for c in range(d))
                    logits.append((j, dot * sc + bias[h, i, j]))
                mx = max(x for _, x in logits)
                den = math.fsum(math.exp(x - mx) for _, x in logits)
                assert abs(LSE[b, h, i] - (mx + math.log(den))) < 1e-13
                for c in range(d):
                    num = math.fsum(math.exp(x - mx) * v[b, h, j, c] for j, x in logits)
                    gate = 1.0 / (1.0 + math.exp(-g[b, h, i, c]))
                    assert abs(O[b, h, i, c] - gate * num / den) < 1e-13


def test_two_key_closed_form():
    """With two keys the softmax is a logistic: P0 = sigmoid(L0 - L1)."""
    rng = np.random.default_rng(3)
    q, k, v, g, dout = (rng.standard_normal((1, 1, 3, 2)) for _ in range(5))
    k = k[:, :, :2]
    v = v[:, :, :2]
    # queries 3, keys 2 is not a square problem; use N=2 for both
    q, g, dout = q[:, :, :2], g[:, :, :2], dout[:, :, :2]
    bias = rng.standard_normal((1, 2, 2))
    O, LSE = oracle.attention_forward(q, k, v, g, bias)
    for i in range(2):
        L = [float(q[0, 0, i] @ k[0, 0, j]) / math.sqrt(2) + bias[0, i, j] for j in range(2)]
        p0 = 1.0 / (1.0 + math.exp(-(L[0] - L[1])))
        for c in range(2):
            A = p0 * v[0, 0, 0, c] + (1 - p0) * v[0, 0, 1, c]
            assert abs(O[0, 0, i, c] - A / (1 + math.exp(-g[0, 0, i, c]))) < 1e-14
        # log(e^a + e^b) = max + log1p(e^-|a-b|)
        assert abs(LSE[0, 0, i] - (max(L) + math.log1p(math.exp(-abs(L[0] - L[1]))))) < 1e-14
    # bias gradient in closed form: dL/dL0 = p0 (1-p0) (dP0 - dP1) for the logistic
    grads = oracle.attention_backward(q, k, v, g, bias, None, dout)
    for i in range(2):
        L = [float(q[0, 0, i] @ k[0, 0, j]) / math.sqrt(2) + bias[0, i, j] for j in range(2)]
        p0 = 1.0 / (1.0 + math.exp(-(L[0] - L[1])))
        s = 1.0 / (1.0 + np.exp(-g[0, 0, i]))
        dA = dout[0, 0, i] * s
        dp0, dp1 = float(dA @ v[0, 0, 0]), float(dA @ v[0, 0, 1])
        expect = p0 * (1 - p0) * (dp0 - dp1)
        assert abs(grads["dbias"][0, i, 0] - expect) < 1e-14
        assert abs(grads["dbias"][0, i, 1] + expect) < 1e-14


# ------------------------------------------------ reductions to known routines

def test_reduces_to_library_attention_when_bias_zero_and_gate_large():
    torch = pytest.importorskip("torch")
    q, k, v, _, _, keep, _ = _tiny(B=3, H=2, N=9, d=5, masked=(0, 4))
    g = np.full(q.shape, 40.0)
    bias = np.zeros((2, 9, 9))
    O, _ = oracle.attention_forward(q, k, v, g, bias, keep)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    mask = torch.from_numpy(keep != 0).view(1, 1, 1, 9).expand(3, 2, 9, 9)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-13)


def test_uniform_case_is_gated_mean_of_kept_values():
    q, k, v, g, bias, keep, _ = _tiny(B=2, H=2, N=6, d=3, masked=(2,))
    z = np.zeros_like(q)
    O, LSE = oracle.attention_forward(z, z, v, g, np.zeros_like(bias), keep)
    mean = v[:, :, keep != 0, :].mean(axis=2, keepdims=True)
    np.testing.assert_allclose(O, oracle.sigmoid(g) * mean, rtol=0, atol=1e-14)
    np.testing.assert_allclose(LSE, math.log(int(keep.sum())), rtol=0, atol=1e-14)


def test_gate_zero_halves_the_output():
    q, k, v, g, bias, keep, _ = _tiny()
    O40, _ = oracle.attention_forward(q, k, v, np.full(q.shape, 40.0), bias, keep)
    O0, _ = oracle.attention_forward(q, k, v, np.zeros(q.shape), bias, keep)
    np.testing.assert_allclose(O0, 0.5 * O40, rtol=0, atol=1e-15)


def test_single_kept_key():
    N = 5
    q, k, v, g, bias, _, dout = _tiny(N=N)
    keep = np.zeros(N, np.uint8)
    keep[3] = 1
    O, LSE = oracle.attention_forward(q, k, v, g, bias, keep)
    np.testing.assert_allclose(O, oracle.sigmoid(g) * v[:, :, 3:4, :], rtol=0, atol=1e-15)
    grads = oracle.attention_backward(q, k, v, g, bias, keep, dout)
    assert np.all(grads["dq"] == 0) and np.all(grads["dk"] == 0)
    assert np.all(grads["dbias"] == 0)


def test_fully_masked_reading():
    q, k, v, g, bias, _, dout = _tiny(N=4)
    keep = np.zeros(4, np.uint8)
    O, LSE = oracle.attention_forward(q, k, v, g, bias, keep)
    assert np.all(O == 0) and np.all(np.isneginf(LSE))
    grads = oracle.attention_backward(q, k, v, g, bias, keep, dout)
    for name in ("dq", "dk", "dv", "dg", "dbias"):
        assert np.all(grads[name] == 0), name


# ---------------------------------------------------------- gradient pins

def _loss_attn(q, k, v, g, bias, keep, dout):
    O, _ = oracle.attention_forward(q, k, v, g, bias, keep)
    return float(np.sum(O * dout))


def test_attention_gradients_match_central_differences():
    q, k, v, g, bias, keep, dout = _tiny(B=2, H=2, N=5, d=3, masked=(3,))
    grads = oracle.attention_backward(q, k, v, g, bias, keep, dout)
    args = {"q": q, "k": k, "v": v, "g": g, "bias": bias}
    h = 1e-6
    for name, x in args.items():
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            fp = _loss_attn(q, k, v, g, bias, keep, dout)
            x[idx] = old - h
            fm = _loss_attn(q, k, v, g, bias, keep, dout)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        ana = grads["d" + name]
        err = np.max(np.abs(num - ana)) / max(1e-12, np.max(np.abs(ana)))
        assert err < 1e-7, (name, err)


def test_bias_gradient_is_dS_summed_over_the_broadcast_axis():
    q, k, v, g, bias, keep, dout = _tiny(B=4, H=2, N=6, d=3, masked=(5,))
    shared = oracle.attention_backward(q, k, v, g, bias, keep, dout)
    expanded_bias = np.broadcast_to(bias, (4,) + bias.shape).copy()
    expanded = oracle.attention_backward(q, k, v, g, expanded_bias, keep, dout)
    assert expanded["dbias"].shape == (4, 2, 6, 6)
    np.testing.assert_allclose(expanded["dbias"].sum(0), shared["dbias"], rtol=1e-13, atol=1e-15)
    # and the per-row bias gradient is the per-row score gradient: rows sum to zero
    np.testing.assert_allclose(expanded["dbias"].sum(-1), 0.0, atol=1e-14)
    for name in ("dq", "dk", "dv", "dg"):
        np.testing.assert_allclose(expanded[name], shared[name], rtol=0, atol=1e-15)


def test_gradient_invariants():
    q, k, v, g, bias, keep, dout = _tiny(B=3, H=2, N=7, d=4, masked=(1, 6))
    gr = oracle.attention_backward(q, k, v, g, bias, keep, dout)
    # Q -> aQ, K -> K/a leaves the logits unchanged, so tr(Q^T dQ) = tr(K^T dK)
    np.testing.assert_allclose(np.sum(q * gr["dq"], axis=(2, 3)), np.sum(k * gr["dk"], axis=(2, 3)),
                               rtol=0, atol=1e-13)
    # a shift of a bias row by a constant does not change O: rows of dBias sum to 0
    np.testing.assert_allclose(gr["dbias"].sum(-1), 0.0, atol=1e-13)
    # masked keys receive exactly zero gradient
    for name in ("dk", "dv"):
        assert np.all(gr[name][:, :, keep == 0, :] == 0.0)
    assert np.all(gr["dbias"][:, :, keep == 0] == 0.0)


def test_identities_used_by_the_gpu_path():
    """dG = dO*O*(1-sigmoid(G)), and sum_j P dP = sum_c dO*O (row statistic D)."""
    q, k, v, g, bias, keep, dout = _tiny(B=2, H=2, N=6, d=4, masked=(2,))
    O, _ = oracle.attention_forward(q, k, v, g, bias, keep)
    gr = oracle.attention_backward(q, k, v, g, bias, keep, dout)
    s = oracle.sigmoid(g)
    np.testing.assert_allclose(gr["dg"], dout * O * (1 - s), rtol=0, atol=1e-14)
    P = _probs(q, k, bias, keep)
    dP = np.matmul(dout * s, np.swapaxes(v, -1, -2))
    np.testing.assert_allclose(np.sum(P * dP, -1), np.sum(dout * O, -1), rtol=0, atol=1e-13)


def test_shift_invariance_of_bias_rows():
    q, k, v, g, bias, keep, _ = _tiny()
    shift = _rand(2, 5, 1)
    O1, L1 = oracle.attention_forward(q, k, v, g, bias, keep)
    O2, L2 = oracle.attention_forward(q, k, v, g, bias + shift, keep)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L2 - L1, np.broadcast_to(shift[None, :, :, 0], L1.shape), atol=1e-13)


# --------------------------------------------------------------- equivariance

def test_key_and_query_permutation_equivariance():
    q, k, v, g, bias, keep, dout = _tiny(B=2, H=2, N=6, d=3, masked=(1,))
    O, L = oracle.attention_forward(q, k, v, g, bias, keep)
    gr = oracle.attention_backward(q, k, v, g, bias, keep, dout)
    pi = np.array([4, 0, 5, 2, 1, 3])
    # keys
    Ok, Lk = oracle.attention_forward(q, k[:, :, pi], v[:, :, pi], g, bias[:, :, pi], keep[pi])
    grk = oracle.attention_backward(q, k[:, :, pi], v[:, :, pi], g, bias[:, :, pi], keep[pi], dout)
    np.testing.assert_allclose(Ok, O, atol=1e-14)
    np.testing.assert_allclose(Lk, L, atol=1e-14)
    np.testing.assert_allclose(grk["dk"], gr["dk"][:, :, pi], atol=1e-14)
    np.testing.assert_allclose(grk["dv"], gr["dv"][:, :, pi], atol=1e-14)
    np.testing.assert_allclose(grk["dbias"], gr["dbias"][:, :, pi], atol=1e-14)
    np.testing.assert_allclose(grk["dq"], gr["dq"], atol=1e-14)
    # queries
    Oq, _ = oracle.attention_forward(q[:, :, pi], k, v, g[:, :, pi], bias[:, pi, :], keep)
    grq = oracle.attention_backward(q[:, :, pi], k, v, g[:, :, pi], bias[:, pi, :], keep, dout[:, :, pi])
    np.testing.assert_allclose(Oq, O[:, :, pi], atol=1e-14)
    np.testing.assert_allclose(grq["dq"], gr["dq"][:, :, pi], atol=1e-14)
    np.testing.assert_allclose(grq["dg"], gr["dg"][:, :, pi], atol=1e-14)
    np.testing.assert_allclose(grq["dbias"], gr["dbias"][:, pi, :], atol=1e-14)
    np.testing.assert_allclose(grq["dk"], gr["dk"], atol=1e-14)


def test_copies_as_batch():
    """One call over B copies equals B calls over one copy; dBias adds up."""
    q, k, v, g, bias, keep, dout = _tiny(B=6, H=2, N=5, d=3, masked=())
    O, L = oracle.attention_forward(q, k, v, g, bias, None)
    gr = oracle.attention_backward(q, k, v, g, bias, None, dout)
    acc = np.zeros_like(bias)
    for b in range(6):
        sl = slice(b, b + 1)
        Ob, Lb = oracle.attention_forward(q[sl], k[sl], v[sl], g[sl], bias, None)
        np.testing.assert_allclose(Ob, O[sl], rtol=0, atol=1e-15)
        acc += oracle.attention_backward(q[sl], k[sl], v[sl], g[sl], bias, None, dout[sl])["dbias"]
    np.testing.assert_allclose(acc, gr["dbias"], rtol=1e-13, atol=1e-15)


def test_chunking_does_not_change_results():
    q, k, v, g, bias, keep, dout = _tiny(B=5, H=2, N=6, d=3, masked=(0,))
    a = oracle.attention_backward(q, k, v, g, bias, keep, dout, chunk=2)
    b = oracle.attention_backward(q, k, v, g, bias, keep, dout, chunk=5)
    for name in a:
        np.testing.assert_allclose(a[name], b[name], rtol=0, atol=1e-14)


# ------------------------------------------------------- pair-weighted average

def _tiny_pwa(S=3, N=5, H=2, d=3, masked=(), seed=5):
    rng = np.random.default_rng(seed)
    b = rng.standard_normal((H, N, N))
    v, g, dout = (rng.standard_normal((S, N, H, d)) for _ in range(3))
    keep = None
    if masked:
        keep = np.ones(N, np.uint8)
        keep[list(masked)] = 0
    return b, v, g, keep, dout


def test_pwa_matches_naive_six_dimensional_form():
    b, v, g, keep, _ = _tiny_pwa(S=2, N=4, H=2, d=3, masked=(1,))
    O, _ = oracle.pwa_forward(b, v, g, keep)
    np.testing.assert_allclose(O, oracle.pwa_forward_naive(b, v, g, keep), rtol=0, atol=1e-14)


@pytest.mark.parametrize("masked", [(), (2,)])
def test_pwa_is_attention_with_zero_query_and_key(masked):
    """Q = K = 0 turns the attention oracle into the pair-weighted average.

    Two independent code paths: the attention oracle on the [B=S, H, N, d]
    layout and the PWA oracle on [S, N, H, d].
    """
    S, N, H, d = 3, 6, 2, 4
    b, v, g, keep, dout = _tiny_pwa(S, N, H, d, masked)
    t = lambda x: np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))  # [S,N,H,d] -> [S,H,N,d]
    z = np.zeros((S, H, N, d))
    Oa, La = oracle.attention_forward(z, z, t(v), t(g), b, keep)
    Op, lse = oracle.pwa_forward(b, v, g, keep)
    np.testing.assert_allclose(t(Op), Oa, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, La[0], rtol=0, atol=1e-14)
    ga = oracle.attention_backward(z, z, t(v), t(g), b, keep, t(dout))
    gp = oracle.pwa_backward(b, v, g, keep, dout)
    np.testing.assert_allclose(t(gp["dv"]), ga["dv"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(t(gp["dg"]), ga["dg"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(gp["db"], ga["dbias"], rtol=0, atol=1e-13)


def test_pwa_gradients_match_central_differences():
    b, v, g, keep, dout = _tiny_pwa(S=2, N=4, H=2, d=3, masked=(0,))
    gr = oracle.pwa_backward(b, v, g, keep, dout)

    def loss():
        O, _ = oracle.pwa_forward(b, v, g, keep)
        return float(np.sum(O * dout))

    h = 1e-6
    for name, x in (("db", b), ("dv", v), ("dg", g)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            fp = loss()
            x[idx] = old - h
            fm = loss()
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        err = np.max(np.abs(num - gr[name])) / max(1e-12, np.max(np.abs(gr[name])))
        assert err < 1e-7, (name, err)


def test_pwa_invariants_and_permutations():
    b, v, g, keep, dout = _tiny_pwa(S=3, N=6, H=2, d=3)
    O, _ = oracle.pwa_forward(b, v, g, keep)
    gr = oracle.pwa_backward(b, v, g, keep, dout)
    np.testing.assert_allclose(gr["db"].sum(-1), 0.0, atol=1e-13)
    pi = np.array([2, 5, 0, 1, 4, 3])
    Oj, _ = oracle.pwa_forward(b[:, :, pi], v[:, pi], g, keep)
    grj = oracle.pwa_backward(b[:, :, pi], v[:, pi], g, keep, dout)
    np.testing.assert_allclose(Oj, O, atol=1e-14)
    np.testing.assert_allclose(grj["dv"], gr["dv"][:, pi], atol=1e-14)
    np.testing.assert_allclose(grj["db"], gr["db"][:, :, pi], atol=1e-14)
    Oi, _ = oracle.pwa_forward(b[:, pi, :], v, g[:, pi], keep)
    gri = oracle.pwa_backward(b[:, pi, :], v, g[:, pi], keep, dout[:, pi])
    np.testing.assert_allclose(Oi, O[:, pi], atol=1e-14)
    np.testing.assert_allclose(gri["dg"], gr["dg"][:, pi], atol=1e-14)
    np.testing.assert_allclose(gri["db"], gr["db"][:, pi, :], atol=1e-14)
    np.testing.assert_allclose(gri["dv"], gr["dv"], atol=1e-14)


def test_pwa_uniform_weights_give_gated_mean():
    b, v, g, _, _ = _tiny_pwa(S=2, N=5, H=3, d=2)
    O, lse = oracle.pwa_forward(np.zeros_like(b), v, g)
    np.testing.assert_allclose(O, oracle.sigmoid(g) * v.mean(axis=1, keepdims=True), atol=1e-15)
    np.testing.assert_allclose(lse, math.log(5), atol=1e-15)


# ---------------------------------------------------------- workload recipe pin

def test_workload_recipe_matches_fixture():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "workloads.json")
    with open(path) as f:
        fixture = json.load(f)
    for name, spec in fixture["configs"].items():
        cfg = workloads.CONFIGS[name]
        for key, val in spec["shape"].items():
            assert getattr(cfg, key) == val, (name, key)
        assert cfg.dtype == spec["dtype"], name
        assert cfg.mask == spec["mask"], name
    for name, spec in fixture["proj_configs"].items():
        cfg = workloads.CONFIGS[name]
        assert cfg.kind == "bias_proj", name
        for key, val in spec["shape"].items():
            assert getattr(cfg, key) == val, (name, key)
    for name, spec in fixture["local_configs"].items():
        cfg = workloads.CONFIGS[name]
        assert cfg.kind == "local_attention" and cfg.mask == spec["mask"], name
        for key, val in spec["shape"].items():
            assert getattr(cfg, key) == val, (name, key)
    lin = workloads.local_inputs(workloads.LocalConfig("small", B=2, H=3, N=70, d=8, mask="tail:5", seed=6))
    assert lin["bias"].shape == (3, 3, 32, 128) and lin["q"].shape == (2, 3, 70, 8)
    assert np.all(lin["key_mask"][65:] == 0) and np.all(lin["key_mask"][:65] == 1)
    small = workloads.ProjConfig("small", N=6, H=3, c=32, seed=5)
    pin = workloads.bias_proj_inputs(small)
    assert pin["z"].shape == (6, 6, 32) and pin["z"].dtype == np.uint16
    assert pin["w"].shape == (3, 32) and pin["w"].dtype == np.float32
    assert pin["dbias"].shape == (3, 6, 6)
    assert np.array_equal(pin["gamma64"], pin["gamma"].astype(np.float64))
    # small configs: check the drawn arrays
    inp = workloads.attention_inputs(workloads.CONFIGS["tiny_fp32"])
    assert inp["q"].shape == (32, 4, 32, 32) and inp["bias"].shape == (4, 32, 32)
    assert int((inp["key_mask"] == 0).sum()) == 3
    tri = workloads.scaled_attention_config(workloads.CONFIGS["tri_attn_n384"], B=2)
    inp = workloads.attention_inputs(tri)
    assert np.all(inp["key_mask"][:365] == 1) and np.all(inp["key_mask"][365:] == 0)
    assert inp["q"].dtype == np.uint16


# ------------------------------------------------------- query-row subsets

def test_query_row_subset_matches_full():
    """The general (Nq != Nk) form on a subset of query rows gives those rows
    of the full result; the dBias rows still sum over every batch row."""
    q, k, v, g, bias, keep, dout = _tiny(B=3, H=2, N=7, d=4, masked=(2,))
    rows = np.array([0, 5, 6])
    O, L = oracle.attention_forward(q, k, v, g, bias, keep)
    gr = oracle.attention_backward(q, k, v, g, bias, keep, dout)
    Os, Ls = oracle.attention_forward(q[:, :, rows], k, v, g[:, :, rows], bias[:, rows], keep)
    grs = oracle.attention_backward(q[:, :, rows], k, v, g[:, :, rows], bias[:, rows], keep,
                                    dout[:, :, rows])
    np.testing.assert_allclose(Os, O[:, :, rows], atol=1e-15)
    np.testing.assert_allclose(Ls, L[:, :, rows], atol=1e-15)
    np.testing.assert_allclose(grs["dq"], gr["dq"][:, :, rows], atol=1e-15)
    np.testing.assert_allclose(grs["dbias"], gr["dbias"][:, rows], atol=1e-14)
    b, v2, g2, keep2, dout2 = _tiny_pwa(S=3, N=8, H=2, d=3, masked=(4,))
    Op, lp = oracle.pwa_forward(b, v2, g2, keep2)
    gp = oracle.pwa_backward(b, v2, g2, keep2, dout2)
    Ops, lps = oracle.pwa_forward(b[:, rows], v2, g2[:, rows], keep2)
    gps = oracle.pwa_backward(b[:, rows], v2, g2[:, rows], keep2, dout2[:, rows])
    np.testing.assert_allclose(Ops, Op[:, rows], atol=1e-15)
    np.testing.assert_allclose(lps, lp[:, rows], atol=1e-15)
    np.testing.assert_allclose(gps["db"], gp["db"][:, rows], atol=1e-14)
    np.testing.assert_allclose(gps["dg"], gp["dg"][:, rows], atol=1e-15)
