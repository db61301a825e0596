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


def check_all(tag: str, pairs: dict, tol: float, floors: dict | None = None) -> dict:
    """Compare every (got, ref) pair, log all relative errors, then assert."""
    floors = floors or {}
    rels = {}
    for name, (got, ref) in pairs.items():
        assert got.shape == ref.shape, (tag, name, got.shape, ref.shape)
        fin_ok = np.array_equal(np.isfinite(got), np.isfinite(ref))
        rels[name] = rel_err(got, ref, floors.get(name, 0.0))[0] if fin_ok else float("nan")
    log(f"{tag}: " + " ".join(f"{k}={v:.2e}" for k, v in rels.items()))
    for name, (got, ref) in pairs.items():
        assert_close(f"{tag} {name}", got, ref, tol, floors.get(name, 0.0))
    return rels
