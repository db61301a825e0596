"""Pair-biased gated attention and MSA pair-weighted averaging for MI355X (gfx950).

The computation lives in libpba.so (hand-written HIP kernels behind the C ABI
in include/pba.h); this package only loads it and marshals torch tensors.
"""
from .ops import (  # noqa: F401
    pba_forward, pba_backward, pba_backward_workspace_bytes,
    pair_weighted_avg, pair_weighted_avg_backward,
    pair_weighted_avg_workspace_bytes, pair_weighted_avg_backward_workspace_bytes,
    pba_backward_timed, pair_weighted_avg_timed, pair_weighted_avg_backward_timed,
)
from ._lib import PbaError, LIB_PATH  # noqa: F401
