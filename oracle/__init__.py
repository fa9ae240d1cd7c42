"""fp64 CPU oracle (test infrastructure only; see nbattn_oracle)."""
from .nbattn_oracle import *  # noqa: F401,F403
