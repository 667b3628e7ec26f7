"""fp64 CPU oracle for the NSA forward pass — test infrastructure only (see nsa_oracle.py)."""
from .nsa_oracle import *  # noqa: F401,F403
from .nsa_oracle import CMP, SEL, LOC, BRANCH_NAMES  # noqa: F401
