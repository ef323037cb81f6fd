"""fp64 CPU oracle (test infrastructure only; see dit_oracle)."""
from .dit_oracle import *  # noqa: F401,F403
from . import dit_oracle  # noqa: F401
