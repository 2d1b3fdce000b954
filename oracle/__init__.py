"""fp64 CPU oracle (test infrastructure only; see harp_oracle)."""
from .harp_oracle import *  # noqa: F401,F403
