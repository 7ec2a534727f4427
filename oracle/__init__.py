"""fp64 CPU oracle (test infrastructure; never used by the product path)."""

from .vsa_oracle import *  # noqa: F401,F403
from .vsa_oracle import __all__  # noqa: F401
