"""Helpers shared by the GPU tests: host <-> device copies and the tolerance check."""
from __future__ import annotations

import sys

import numpy as np

import workloads

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dtype: str):
    import torch
    if arr.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(arr)).cuda()
    if dtype == "bf16":
        assert arr.dtype == np.uint16
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return workloads.bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return workloads.bf16_bits_to_f32(bits).astype(np.float64)
    return bits.astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray, floor: float = 0.0):
    """(max |got - ref| / max(max |ref|, floor), max |got - ref|) over finite entries."""
    fin = np.isfinite(ref)
    g, r = got[fin], ref[fin]
    if r.size == 0:
        return 0.0, 0.0
    scale = max(float(np.max(np.abs(r))), floor)
    err = float(np.max(np.abs(g - r)))
    return (err / scale if scale > 0 else (0.0 if err == 0 else float("inf"))), err


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, tol: float, floor: float = 0.0) -> float:
    """max |got - ref| <= tol * max |ref| over the whole tensor (the parity bar).

    floor: where the exact reference is identically zero (a gradient that
    vanishes analytically), the bar is taken relative to `floor`, the natural
    magnitude of that gradient; 0 keeps the bar exact.
    """
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: non-finite pattern differs"
    if not fin.all():
        assert np.array_equal(got[~fin], ref[~fin]), f"{name}: non-finite values differ"
    rel, err = rel_err(got, ref, floor)
    assert rel <= tol, f"{name}: max|err| = {err:.3e} = {rel:.3e} * scale > {tol:.1e}"
    return rel


def check_all(tag: str, pairs: dict, tol: float, floors: dict | None = None, rerun=None) -> dict:
    """Compare every (got, ref) pair, log all relative errors, then assert.

    rerun: optional callable for the bf16 backward.  Given the names that
    fail the bar, it returns (grads, bounds): those gradients recomputed by
    the GPU backward from the oracle's forward output O rounded to bf16 (and
    the oracle's lse) instead of the GPU forward's, and elementwise bounds on
    the error that storing O in bf16 forces into them (`d_rounding_slack`).
    Such a tensor passes if |grad - ref| <= tol * max|ref| + bound
    everywhere.  Only dq, dk and dbias qualify: they depend on O through
    D = rowsum(dO * O), and when dS is a small difference of large terms
    (two keys) the rounding of O to bf16 alone moves them past the bar.
    """
    floors = floors or {}
    rels = {}
    for name, (got, ref) in pairs.items():
        assert got.shape == ref.shape, (tag, name, got.shape, ref.shape)
        fin_ok = np.array_equal(np.isfinite(got), np.isfinite(ref))
        rels[name] = rel_err(got, ref, floors.get(name, 0.0))[0] if fin_ok else float("nan")
    log(f"{tag}: " + " ".join(f"{k}={v:.2e}" for k, v in rels.items()))
    failing = [n for n, r in rels.items() if not r <= tol and n in ("dq", "dk", "dbias")]
    regot, bounds = rerun(failing) if (rerun is not None and failing) else ({}, {})
    for name, (got, ref) in pairs.items():
        if name in bounds:
            got = regot[name]
            fin = np.isfinite(ref)
            assert np.array_equal(np.isfinite(got), fin), f"{tag} {name}: non-finite pattern differs"
            err = np.abs(got - ref)[fin]
            bar = tol * float(np.max(np.abs(ref[fin]))) + bounds[name][fin]
            worst = float(np.max(err / bar))
            log(f"{tag} {name}: {rels[name]:.2e} of max|ref| end to end; from the oracle's bf16 O: "
                f"{float(np.max(err)) / float(np.max(np.abs(ref[fin]))):.2e} of max|ref|, "
                f"max err / (tol*max|ref| + O-storage bound) = {worst:.2f}")
            assert worst <= 1.0, f"{tag} {name}: error exceeds tol*max|ref| + O-storage bound ({worst:.2f})"
        else:
            assert_close(f"{tag} {name}", got, ref, tol, floors.get(name, 0.0))
    return rels


def bf16_round_f64(x: np.ndarray) -> np.ndarray:
    """float64 values rounded to bf16 (through float32, nearest even), as float64."""
    return workloads.bf16_bits_to_f32(workloads.bf16_round_bits(x.astype(np.float32))).astype(np.float64)


def oracle_probs(forward, inp) -> np.ndarray:
    """The oracle's attention probabilities P [B,H,N,N] (key axis last), read
    off the oracle's own forward pass: with the gate at G = 40 (sigmoid(40)
    is 1.0 in float64) and V one-hot over a chunk of d keys, the output's
    channel c is P at key c0 + c.  `forward(v, g)` runs the oracle forward on
    the case's other inputs.  Small cases only."""
    q = inp["q64"]
    B, H, N, d = q.shape
    P = np.zeros((B, H, N, N))
    g40 = np.full(q.shape, 40.0)
    for c0 in range(0, N, d):
        n = min(d, N - c0)
        v = np.zeros(q.shape)
        v[:, :, np.arange(c0, c0 + n), np.arange(n)] = 1.0
        O, _ = forward(v, g40)
        P[..., c0:c0 + n] = O[..., :n]
    return P


def d_rounding_slack(inp, O_ref, P, scale) -> dict:
    """Elementwise bounds on the backward error that storing the forward
    output O in bf16 forces.

    The backward receives O only in its storage type and forms
    D_i = sum_c dO_ic O_ic from it (the identity D_i = sum_j P_ij dP_ij,
    pinned in the oracle tests); rounding O to bf16 shifts D_i by
    dD_i = sum_c dO_ic (bf16(O_ic) - O_ic), computed here from the oracle's
    own O.  That shifts dS_ij by -P_ij dD_i, so dq_i moves by at most
    scale |dD_i| sum_j P_ij |K_j|, dk_j by scale sum_i P_ij |dD_i| |Q_i| and
    dbias_ij by sum_b P_bij |dD_bi| (dense bias layout [H,N,N]).
    """
    dD = np.abs(np.sum(inp["dout64"] * (bf16_round_f64(O_ref) - O_ref), axis=-1))  # [B,H,N]
    k, q = np.abs(inp["k64"]), np.abs(inp["q64"])
    return {
        "dq": scale * dD[..., None] * np.matmul(P, k),
        "dk": scale * np.matmul(np.swapaxes(P, -1, -2), dD[..., None] * q),
        "dbias": np.sum(P * dD[..., None], axis=0),
    }
