"""CPU oracle (test infrastructure only; see sage_oracle's header)."""
from .sage_oracle import *  # noqa: F401,F403
