"""CPU oracle (test infrastructure only; see tq_oracle)."""
from .tq_oracle import *  # noqa: F401,F403
