"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""

from .norm_oracle import *  # noqa: F401,F403
from .norm_oracle import __all__ as _norm_all
from .pack_oracle import *  # noqa: F401,F403
from .pack_oracle import __all__ as _pack_all
from .rope_oracle import *  # noqa: F401,F403
from .rope_oracle import __all__ as _rope_all

__all__ = list(_rope_all) + list(_norm_all) + list(_pack_all)
