"""PyTorch-facing wrappers with the names of the C ABI.

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in libpba's kernels.  Layouts (contiguous, row-major):
  attention  q, k, v, g, out, dout, dq, dk, dv, dg: [B, H, N, d]; bias, dbias: [H, N, N]
  pair-bias projection  z, dz: [N, N, c] bf16; gamma, beta: [c], w: [H, c] float32; bias: [H, N, N]
  windowed attention  q, k, v, g, out, ...: [B, H, N, d]; bias, dbias: [H, ceil(N/32), 32, 128]
  pair-weighted average  v, g, out, dout, dv, dg: [S, N, H, d]; b, db: [H, N, N]
  key_mask: [N] uint8 (0 = masked) or None.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_DT = {torch.float32: _lib.PBA_F32, torch.bfloat16: _lib.PBA_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _check_tensors(ref: torch.Tensor, named: dict, shapes: dict):
    if ref.dtype not in _DT:
        raise TypeError(f"unsupported dtype {ref.dtype}")
    if ref.device.type != "cuda":
        raise ValueError("pba kernels run on the GPU; got a tensor on " + str(ref.device))
    for name, t in named.items():
        if t is None:
            continue
        want_dtype = torch.uint8 if name == "key_mask" else (torch.float32 if name.startswith("lse") else ref.dtype)
        if t.dtype != want_dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {want_dtype}")
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if name in shapes and tuple(t.shape) != tuple(shapes[name]):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shapes[name])}")


def pba_forward(q, k, v, g, bias, key_mask=None):
    """Pair-biased gated attention forward; returns (out, lse)."""
    lib = _lib.load()
    B, H, N, d = q.shape
    shp = {"q": (B, H, N, d), "k": (B, H, N, d), "v": (B, H, N, d), "g": (B, H, N, d),
           "bias": (H, N, N), "key_mask": (N,)}
    _check_tensors(q, dict(q=q, k=k, v=v, g=g, bias=bias, key_mask=key_mask), shp)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = lib.pba_forward(B, H, N, d, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bias),
                         _ptr(key_mask), _ptr(out), _ptr(lse), _stream(q.device))
    _lib.check("pba_forward", st)
    return out, lse


def pba_backward_workspace_bytes(B, H, N, d, dtype) -> int:
    return int(_lib.load().pba_backward_workspace_bytes(B, H, N, d, _DT[dtype]))


def pba_backward(q, k, v, g, bias, key_mask, out, lse, dout, workspace=None):
    """Backward; returns dict(dq, dk, dv, dg, dbias).  dbias is summed over B."""
    lib = _lib.load()
    B, H, N, d = q.shape
    shp = {n: (B, H, N, d) for n in ("q", "k", "v", "g", "out", "dout")}
    shp.update(bias=(H, N, N), key_mask=(N,), lse=(B, H, N))
    _check_tensors(q, dict(q=q, k=k, v=v, g=g, bias=bias, key_mask=key_mask, out=out, lse=lse,
                           dout=dout), shp)
    nbytes = lib.pba_backward_workspace_bytes(B, H, N, d, _DT[q.dtype])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dq, dk, dv, dg = (torch.empty_like(q) for _ in range(4))
    dbias = torch.empty_like(bias)
    st = lib.pba_backward(B, H, N, d, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bias),
                          _ptr(key_mask), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(dg), _ptr(dbias), _ptr(workspace), workspace.numel(),
                          _stream(q.device))
    _lib.check("pba_backward", st)
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dbias": dbias}


def pba_backward_noalloc(q, k, v, g, bias, key_mask, out, lse, dout, grads=None):
    """Backward without a workspace: the library's static scratch area takes
    its place (see include/pba.h).  With `grads` (a dict of preallocated dq,
    dk, dv, dg, dbias) nothing is allocated on the call path; otherwise the
    gradients are allocated here.  Returns the dict of gradients."""
    lib = _lib.load()
    B, H, N, d = q.shape
    shp = {n: (B, H, N, d) for n in ("q", "k", "v", "g", "out", "dout", "dq", "dk", "dv", "dg")}
    shp.update(bias=(H, N, N), dbias=(H, N, N), key_mask=(N,), lse=(B, H, N))
    if grads is None:
        grads = {n: torch.empty_like(q) for n in ("dq", "dk", "dv", "dg")}
        grads["dbias"] = torch.empty_like(bias)
    _check_tensors(q, dict(q=q, k=k, v=v, g=g, bias=bias, key_mask=key_mask, out=out, lse=lse,
                           dout=dout, **grads), shp)
    st = lib.pba_backward_noalloc(B, H, N, d, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bias),
                                  _ptr(key_mask), _ptr(out), _ptr(lse), _ptr(dout), _ptr(grads["dq"]),
                                  _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dg"]), _ptr(grads["dbias"]),
                                  _stream(q.device))
    _lib.check("pba_backward_noalloc", st)
    return grads


def pair_weighted_avg_workspace_bytes(S, N, H, d, dtype) -> int:
    return int(_lib.load().pair_weighted_avg_workspace_bytes(S, N, H, d, _DT[dtype]))


def pair_weighted_avg(b, v, g, key_mask=None, workspace=None):
    """MSA pair-weighted average forward; returns (out, lse_w)."""
    lib = _lib.load()
    S, N, H, d = v.shape
    _check_tensors(v, dict(b=b, v=v, g=g, key_mask=key_mask),
                   {"b": (H, N, N), "v": (S, N, H, d), "g": (S, N, H, d), "key_mask": (N,)})
    nbytes = lib.pair_weighted_avg_workspace_bytes(S, N, H, d, _DT[v.dtype])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=v.device)
    out = torch.empty_like(v)
    lse_w = torch.empty((H, N), dtype=torch.float32, device=v.device)
    st = lib.pair_weighted_avg(S, N, H, d, _DT[v.dtype], _ptr(b), _ptr(key_mask), _ptr(v), _ptr(g),
                               _ptr(out), _ptr(lse_w), _ptr(workspace), workspace.numel(),
                               _stream(v.device))
    _lib.check("pair_weighted_avg", st)
    return out, lse_w


def pair_weighted_avg_backward_workspace_bytes(S, N, H, d, dtype) -> int:
    return int(_lib.load().pair_weighted_avg_backward_workspace_bytes(S, N, H, d, _DT[dtype]))


def pair_weighted_avg_backward(b, v, g, key_mask, out, lse_w, dout, workspace=None):
    """Backward of the pair-weighted average; returns dict(dv, dg, db)."""
    lib = _lib.load()
    S, N, H, d = v.shape
    shp = {n: (S, N, H, d) for n in ("v", "g", "out", "dout")}
    shp.update(b=(H, N, N), key_mask=(N,), lse_w=(H, N))
    _check_tensors(v, dict(b=b, v=v, g=g, key_mask=key_mask, out=out, lse_w=lse_w, dout=dout), shp)
    nbytes = lib.pair_weighted_avg_backward_workspace_bytes(S, N, H, d, _DT[v.dtype])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=v.device)
    dv, dg = torch.empty_like(v), torch.empty_like(g)
    db = torch.empty_like(b)
    st = lib.pair_weighted_avg_backward(S, N, H, d, _DT[v.dtype], _ptr(b), _ptr(key_mask), _ptr(v),
                                        _ptr(g), _ptr(out), _ptr(lse_w), _ptr(dout), _ptr(dv), _ptr(dg),
                                        _ptr(db), _ptr(workspace), workspace.numel(), _stream(v.device))
    _lib.check("pair_weighted_avg_backward", st)
    return {"dv": dv, "dg": dg, "db": db}


def _check_proj(z, params: dict, planes: dict):
    """z [N, N, c] bf16; float32 parameters; bf16 [H, N, N] planes; all on z's device, contiguous."""
    if z.dtype != torch.bfloat16:
        raise TypeError(f"z has dtype {z.dtype}; the projection takes bfloat16 z")
    if z.device.type != "cuda":
        raise ValueError("pba kernels run on the GPU; got a tensor on " + str(z.device))
    if z.dim() != 3 or z.shape[0] != z.shape[1]:
        raise ValueError(f"z must be [N, N, c], got {tuple(z.shape)}")
    for group, dtype in ((params, torch.float32), (planes, torch.bfloat16)):
        for name, (t, shape) in group.items():
            if t.dtype != dtype:
                raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
            if t.device != z.device:
                raise ValueError(f"{name} is on {t.device}, expected {z.device}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
            if tuple(t.shape) != tuple(shape):
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not z.is_contiguous():
        raise ValueError("z must be contiguous")


def pba_bias_proj_forward(z, gamma, beta, w, eps=1e-5):
    """Pair-bias projection bias [H, N, N] (bf16) = Linear(LayerNorm(z)) for z [N, N, c] (bf16);
    gamma, beta [c] and w [H, c] are float32."""
    lib = _lib.load()
    N, c = z.shape[0], z.shape[-1]
    H = w.shape[0]
    _check_proj(z, {"gamma": (gamma, (c,)), "beta": (beta, (c,)), "w": (w, (H, c))}, {})
    bias = torch.empty((H, N, N), dtype=torch.bfloat16, device=z.device)
    st = lib.pba_bias_proj_forward(N, H, c, _lib.PBA_BF16, _ptr(z), _ptr(gamma), _ptr(beta), _ptr(w), float(eps),
                                   _ptr(bias), _stream(z.device))
    _lib.check("pba_bias_proj_forward", st)
    return bias


def pba_bias_proj_backward_workspace_bytes(N, H, c, dtype=torch.bfloat16) -> int:
    return int(_lib.load().pba_bias_proj_backward_workspace_bytes(N, H, c, _DT[dtype]))


def pba_bias_proj_backward(z, gamma, beta, w, dbias, eps=1e-5, workspace=None):
    """Backward of pba_bias_proj_forward; returns dict(dz, dgamma, dbeta, dw)."""
    lib = _lib.load()
    N, c = z.shape[0], z.shape[-1]
    H = w.shape[0]
    _check_proj(z, {"gamma": (gamma, (c,)), "beta": (beta, (c,)), "w": (w, (H, c))},
                {"dbias": (dbias, (H, N, N))})
    nbytes = lib.pba_bias_proj_backward_workspace_bytes(N, H, c, _lib.PBA_BF16)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=z.device)
    dz = torch.empty_like(z)
    dgamma, dbeta, dw = torch.empty_like(gamma), torch.empty_like(beta), torch.empty_like(w)
    st = lib.pba_bias_proj_backward(N, H, c, _lib.PBA_BF16, _ptr(z), _ptr(gamma), _ptr(beta), _ptr(w), float(eps),
                                    _ptr(dbias), _ptr(dz), _ptr(dgamma), _ptr(dbeta), _ptr(dw), _ptr(workspace),
                                    workspace.numel(), _stream(z.device))
    _lib.check("pba_bias_proj_backward", st)
    return {"dz": dz, "dgamma": dgamma, "dbeta": dbeta, "dw": dw}


def local_bias_shape(H, N):
    """Shape of the windowed attention's bias: [H, ceil(N/32), 32, 128]."""
    return (H, (N + 31) // 32, 32, 128)


def pba_local_forward(q, k, v, g, bias, key_mask=None):
    """Windowed pair-biased gated attention forward (bf16, d <= 32); returns (out, lse)."""
    lib = _lib.load()
    B, H, N, d = q.shape
    shp = {"q": (B, H, N, d), "k": (B, H, N, d), "v": (B, H, N, d), "g": (B, H, N, d),
           "bias": local_bias_shape(H, N), "key_mask": (N,)}
    _check_tensors(q, dict(q=q, k=k, v=v, g=g, bias=bias, key_mask=key_mask), shp)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = lib.pba_local_forward(B, H, N, d, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bias),
                               _ptr(key_mask), _ptr(out), _ptr(lse), _stream(q.device))
    _lib.check("pba_local_forward", st)
    return out, lse


def pba_local_backward_workspace_bytes(B, H, N, d, dtype=torch.bfloat16) -> int:
    return int(_lib.load().pba_local_backward_workspace_bytes(B, H, N, d, _DT[dtype]))


def pba_local_backward(q, k, v, g, bias, key_mask, out, lse, dout, workspace=None):
    """Backward of pba_local_forward; returns dict(dq, dk, dv, dg, dbias), dbias summed over B."""
    lib = _lib.load()
    B, H, N, d = q.shape
    shp = {n: (B, H, N, d) for n in ("q", "k", "v", "g", "out", "dout")}
    shp.update(bias=local_bias_shape(H, N), key_mask=(N,), lse=(B, H, N))
    _check_tensors(q, dict(q=q, k=k, v=v, g=g, bias=bias, key_mask=key_mask, out=out, lse=lse,
                           dout=dout), shp)
    nbytes = lib.pba_local_backward_workspace_bytes(B, H, N, d, _DT[q.dtype])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv, dg = (torch.empty_like(q) for _ in range(4))
    dbias = torch.empty_like(bias)
    st = lib.pba_local_backward(B, H, N, d, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bias),
                                _ptr(key_mask), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(dg), _ptr(dbias), _ptr(workspace), workspace.numel(), _stream(q.device))
    _lib.check("pba_local_backward", st)
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dbias": dbias}


# ---- measurement entry points (create HIP events and synchronise) ----------

def _timed_call(fn_name, args):
    lib = _lib.load()
    cap = 8
    ms = (ctypes.c_float * cap)()
    n = ctypes.c_int(0)
    st = getattr(lib, fn_name)(*args, ctypes.cast(ms, ctypes.c_void_p), cap, ctypes.cast(ctypes.pointer(n), ctypes.c_void_p))
    _lib.check(fn_name, st)
    return [float(ms[i]) for i in range(min(n.value, cap))]


def pba_backward_timed(q, k, v, g, bias, key_mask, out, lse, dout, workspace, grads):
    """pba_backward into preallocated `grads` (dq, dk, dv, dg, dbias); returns per-kernel ms."""
    B, H, N, d = q.shape
    return _timed_call("pba_backward_timed", [
        B, H, N, d, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bias), _ptr(key_mask), _ptr(out),
        _ptr(lse), _ptr(dout), _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dg"]),
        _ptr(grads["dbias"]), _ptr(workspace), workspace.numel(), _stream(q.device)])


def pair_weighted_avg_timed(b, v, g, key_mask, out, lse_w, workspace):
    """pair_weighted_avg into preallocated out / lse_w; returns per-kernel ms."""
    S, N, H, d = v.shape
    return _timed_call("pair_weighted_avg_timed", [
        S, N, H, d, _DT[v.dtype], _ptr(b), _ptr(key_mask), _ptr(v), _ptr(g), _ptr(out), _ptr(lse_w),
        _ptr(workspace), workspace.numel(), _stream(v.device)])


def pair_weighted_avg_backward_timed(b, v, g, key_mask, out, lse_w, dout, workspace, grads):
    """pair_weighted_avg_backward into preallocated `grads` (dv, dg, db); returns per-kernel ms."""
    S, N, H, d = v.shape
    return _timed_call("pair_weighted_avg_backward_timed", [
        S, N, H, d, _DT[v.dtype], _ptr(b), _ptr(key_mask), _ptr(v), _ptr(g), _ptr(out), _ptr(lse_w), _ptr(dout),
        _ptr(grads["dv"]), _ptr(grads["dg"]), _ptr(grads["db"]), _ptr(workspace), workspace.numel(),
        _stream(v.device)])


def pba_bias_proj_forward_timed(z, gamma, beta, w, eps, bias):
    """pba_bias_proj_forward into a preallocated bias; returns per-kernel ms."""
    N, c = z.shape[0], z.shape[-1]
    H = w.shape[0]
    return _timed_call("pba_bias_proj_forward_timed", [
        N, H, c, _lib.PBA_BF16, _ptr(z), _ptr(gamma), _ptr(beta), _ptr(w), float(eps), _ptr(bias),
        _stream(z.device)])


def pba_bias_proj_backward_timed(z, gamma, beta, w, dbias, eps, workspace, grads):
    """pba_bias_proj_backward into preallocated `grads` (dz, dgamma, dbeta, dw); returns per-kernel ms."""
    N, c = z.shape[0], z.shape[-1]
    H = w.shape[0]
    return _timed_call("pba_bias_proj_backward_timed", [
        N, H, c, _lib.PBA_BF16, _ptr(z), _ptr(gamma), _ptr(beta), _ptr(w), float(eps), _ptr(dbias),
        _ptr(grads["dz"]), _ptr(grads["dgamma"]), _ptr(grads["dbeta"]), _ptr(grads["dw"]), _ptr(workspace),
        workspace.numel(), _stream(z.device)])


def pba_local_forward_timed(q, k, v, g, bias, key_mask, out, lse):
    """pba_local_forward into preallocated out / lse; returns per-kernel ms."""
    B, H, N, d = q.shape
    return _timed_call("pba_local_forward_timed", [
        B, H, N, d, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bias), _ptr(key_mask), _ptr(out),
        _ptr(lse), _stream(q.device)])


def pba_local_backward_timed(q, k, v, g, bias, key_mask, out, lse, dout, workspace, grads):
    """pba_local_backward into preallocated `grads` (dq, dk, dv, dg, dbias); returns per-kernel ms."""
    B, H, N, d = q.shape
    return _timed_call("pba_local_backward_timed", [
        B, H, N, d, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bias), _ptr(key_mask), _ptr(out),
        _ptr(lse), _ptr(dout), _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dg"]),
        _ptr(grads["dbias"]), _ptr(workspace), workspace.numel(), _stream(q.device)])
