"""CPU oracle (test infrastructure only; see mmsa_oracle.py)."""
from .mmsa_oracle import *  # noqa: F401,F403
