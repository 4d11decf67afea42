"""CPU oracle for the TTQ hot path (test infrastructure only; see ttq_oracle)."""
from .ttq_oracle import *  # noqa: F401,F403
from .ttq_oracle import __all__  # noqa: F401
