"""fp64 CPU oracle (test infrastructure; see hc_oracle's module docstring)."""
from .hc_oracle import *  # noqa: F401,F403
