"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .qi_oracle import *  # noqa: F401,F403
