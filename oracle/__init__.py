"""CPU oracle (test infrastructure only; see twell_oracle's header)."""
from .twell_oracle import *  # noqa: F401,F403
from . import twell_oracle  # noqa: F401
