"""CPU oracle package -- test infrastructure only (see dsv4_oracle)."""
from .dsv4_oracle import *  # noqa: F401,F403
