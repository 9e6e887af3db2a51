"""CPU oracle for the Jano hot path (test infrastructure; see jano_oracle)."""
from .jano_oracle import *  # noqa: F401,F403
