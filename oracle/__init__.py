"""fp64 CPU oracle (test infrastructure; see pba_oracle's header)."""
from .pba_oracle import *  # noqa: F401,F403
from .pba_oracle import __all__  # noqa: F401
