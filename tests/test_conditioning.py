"""Why the two-key bf16 parity cases are expected failures (CPU only).

With two keys, dS_i1 = P_i1 P_i2 (dP_i1 - dP_i2) = -dS_i2 is a small
difference of large terms.  A bf16 backward must round dA = dO * sigmoid(G)
to bf16 (it is a matrix-core operand of dP = dA V^T), and receives the
forward output O in bf16 (the output type), from which it forms
D = rowsum(dO * O).  This test takes the same two-key case as the GPU parity
test, runs the backward chain in float64 with exactly those two roundings and
nothing else, and shows that dq alone moves past the 2e-2 bar, while the same
chain without the roundings matches the oracle to 1e-14.
"""
import math

import numpy as np

import oracle
import workloads


def _bf16(x):
    return workloads.bf16_bits_to_f32(workloads.bf16_round_bits(x.astype(np.float32))).astype(np.float64)


def _dq_with(inp, O, round_da, round_o):
    q, k, v, g, bias, do = (inp[n + "64"] for n in ("q", "k", "v", "g", "bias", "dout"))
    d = q.shape[-1]
    _, L = oracle.attention_forward(q, k, v, g, bias, None)
    P = np.exp(np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(d) + bias - L[..., None])
    dA = do * oracle.sigmoid(g)
    dA = _bf16(dA) if round_da else dA
    Ob = _bf16(O) if round_o else O
    dS = P * (np.matmul(dA, np.swapaxes(v, -1, -2)) - np.sum(do * Ob, axis=-1, keepdims=True))
    return np.matmul(dS, k) / math.sqrt(d)


def test_two_key_backward_is_ill_conditioned_in_bf16():
    cfg = workloads.AttnConfig("case", B=1, H=1, N=2, d=8, dtype="bf16", mask="none", seed=9)
    inp = workloads.attention_inputs(cfg)
    O, _ = oracle.attention_forward(inp["q64"], inp["k64"], inp["v64"], inp["g64"], inp["bias64"], None)
    ref = oracle.attention_backward(inp["q64"], inp["k64"], inp["v64"], inp["g64"], inp["bias64"], None,
                                    inp["dout64"])["dq"]
    scale = np.max(np.abs(ref))
    rel = lambda x: float(np.max(np.abs(x - ref)) / scale)
    assert rel(_dq_with(inp, O, False, False)) < 1e-12
    assert rel(_dq_with(inp, O, True, False)) > 2e-2   # dA rounding alone
    assert rel(_dq_with(inp, O, False, True)) > 2e-2   # O rounding alone
    assert 0.08 < rel(_dq_with(inp, O, True, True)) < 0.12
