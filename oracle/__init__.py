"""fp64 CPU oracle of the CSA2 layer step (test infrastructure only)."""
from .csa2_oracle import *  # noqa: F401,F403
from . import csa2_oracle as core  # noqa: F401
