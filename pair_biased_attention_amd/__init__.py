"""Pair-biased gated attention, MSA pair-weighted averaging and the pair-bias
projection Linear(LayerNorm(z)), and windowed (atom) attention for MI355X (gfx950).

The computation lives in libpba.so (hand-written HIP kernels behind the C ABI
in include/pba.h); this package only loads it and marshals torch tensors.
"""
from .ops import (  # noqa: F401
    pba_forward, pba_backward, pba_backward_workspace_bytes, pba_backward_noalloc,
    pair_weighted_avg, pair_weighted_avg_backward,
    pair_weighted_avg_workspace_bytes, pair_weighted_avg_backward_workspace_bytes,
    pba_backward_timed, pair_weighted_avg_timed, pair_weighted_avg_backward_timed,
    pba_bias_proj_forward, pba_bias_proj_backward, pba_bias_proj_backward_workspace_bytes,
    pba_bias_proj_forward_timed, pba_bias_proj_backward_timed,
    pba_local_forward, pba_local_backward, pba_local_backward_workspace_bytes, local_bias_shape,
    pba_local_forward_timed, pba_local_backward_timed,
)
from ._lib import PbaError, LIB_PATH  # noqa: F401
