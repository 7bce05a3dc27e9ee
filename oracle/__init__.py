"""CPU oracle (test infrastructure only; see oracle.c)."""
from .oracle import *  # noqa: F401,F403
