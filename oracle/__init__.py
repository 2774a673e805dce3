"""CPU oracle (fp64 NumPy) for the block-sparse attention rank share.

Test infrastructure only: the tests, the smoke check and the benchmark's CPU-baseline leg use it; the
HIP library and its Python binding never import it.
"""
from .sparsp_oracle import *  # noqa: F401,F403
