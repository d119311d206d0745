"""CPU oracle (test infrastructure only): see csa_oracle.py."""
from .csa_oracle import *  # noqa: F401,F403
