"""CPU oracle (test infrastructure only; see kk_oracle's module docstring)."""
from .kk_oracle import *  # noqa: F401,F403
