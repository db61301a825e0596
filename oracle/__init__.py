"""fp64 CPU oracle (test infrastructure; see pba_oracle's header)."""
from .pba_oracle import *  # noqa: F401,F403
from .bias_proj_oracle import *  # noqa: F401,F403
from .local_attn_oracle import *  # noqa: F401,F403
from . import pba_oracle as _pba, bias_proj_oracle as _bp, local_attn_oracle as _la

__all__ = list(_pba.__all__) + list(_bp.__all__) + list(_la.__all__)
