"""fp64 CPU oracle for exact scaled dot-product attention (test infrastructure only).

Only the test suite, the package smoke check and the bench's CPU-baseline leg
may import this package; the HIP library and its Python binding never do.
"""
from .sdpa_oracle import *  # noqa: F401,F403
