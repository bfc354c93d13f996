"""CPU oracle (test infrastructure only): see flux3_oracle's header."""
from .flux3_oracle import *  # noqa: F401,F403
from . import flux3_oracle  # noqa: F401
