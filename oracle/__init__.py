"""fp64 CPU oracle (test infrastructure only; see gq_oracle's header)."""
from .gq_oracle import *  # noqa: F401,F403
