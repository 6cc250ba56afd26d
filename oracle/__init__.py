"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""

from .rope_oracle import *  # noqa: F401,F403
from .rope_oracle import __all__  # noqa: F401
