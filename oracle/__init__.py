"""CPU oracle for the GQE attention layer (test infrastructure only)."""
from .gqe_oracle import *  # noqa: F401,F403
from .gqe_oracle import __all__  # noqa: F401
