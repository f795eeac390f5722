"""CPU fp64 oracle of the sparse + low-rank linear layer (test infrastructure only;
the product path never imports it)."""
from .hss_oracle import *  # noqa: F401,F403
from .hss_oracle import TOL, F32, BF16  # noqa: F401
