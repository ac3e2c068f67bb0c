"""fp64 CPU oracle of the Parallel Transformer Block layer.

TEST INFRASTRUCTURE: only the tests, the package smoke entry and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library.
"""
from .ptb_oracle import *  # noqa: F401,F403
