"""fp64 CPU oracle of the Representation Shift hot path (test infrastructure only)."""
from .rs_oracle import *  # noqa: F401,F403
