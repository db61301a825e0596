"""ctypes view of libpba.so (the C ABI declared in include/pba.h).

Only argument marshalling lives here.  There is no fallback: if the library
is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PBA_LIB", os.path.join(_HERE, "lib", "libpba.so"))

PBA_F32 = 0
PBA_BF16 = 1

STATUS = {
    0: "PBA_OK", 1: "PBA_ERR_NULL", 2: "PBA_ERR_SHAPE", 3: "PBA_ERR_UNSUPPORTED",
    4: "PBA_ERR_ALIGN", 5: "PBA_ERR_WORKSPACE", 6: "PBA_ERR_HIP", 7: "PBA_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 128 << 20

# exported symbol -> (restype, argtypes)
_i, _sz, _p, _fl = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
SIGNATURES = {
    "pba_abi_version": (_i, []),
    "pba_status_string": (ctypes.c_char_p, [_i]),
    "pba_forward": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "pba_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "pba_backward": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                          _p, _p, _p, _p, _p, _p, _sz, _p]),
    "pair_weighted_avg_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "pair_weighted_avg": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "pair_weighted_avg_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "pair_weighted_avg_backward": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p,
                                        _p, _p, _p, _p, _sz, _p]),
    "pba_backward_timed": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                _p, _p, _p, _p, _p, _p, _sz, _p, _p, _i, _p]),
    "pair_weighted_avg_timed": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _sz, _p,
                                     _p, _i, _p]),
    "pair_weighted_avg_backward_timed": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p,
                                              _p, _p, _p, _p, _sz, _p, _p, _i, _p]),
    "pba_bias_proj_forward": (_i, [_i, _i, _i, _i, _p, _p, _p, _p, _fl, _p, _p]),
    "pba_bias_proj_backward_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "pba_bias_proj_backward": (_i, [_i, _i, _i, _i, _p, _p, _p, _p, _fl, _p, _p, _p, _p, _p,
                                    _p, _sz, _p]),
    "pba_bias_proj_forward_timed": (_i, [_i, _i, _i, _i, _p, _p, _p, _p, _fl, _p, _p, _p, _i, _p]),
    "pba_bias_proj_backward_timed": (_i, [_i, _i, _i, _i, _p, _p, _p, _p, _fl, _p, _p, _p, _p, _p,
                                          _p, _sz, _p, _p, _i, _p]),
    "pba_local_forward": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "pba_local_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "pba_local_backward": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                _p, _p, _p, _p, _p, _p, _sz, _p]),
    "pba_local_forward_timed": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                     _p, _i, _p]),
    "pba_local_backward_timed": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                      _p, _p, _p, _p, _p, _p, _sz, _p, _p, _i, _p]),
    "pba_backward_noalloc": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                  _p, _p, _p, _p, _p, _p]),
}

_lib = None


class PbaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = STATUS.get(status, f"status {status}")
        if _lib is not None:
            try:
                msg = _lib.pba_status_string(status).decode()
            except Exception:  # pragma: no cover
                pass
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


def load(path: str | None = None):
    """Load libpba.so once and declare every exported signature."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libpba.so not found at {p}; build it with "
                           "`python -m pair_biased_attention_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        raise PbaError(fn, status)
