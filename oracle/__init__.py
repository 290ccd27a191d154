"""CPU oracle for blockwise low-bit compression -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) must never
import it.  See ``oracle/lowbit_oracle.c`` for what is computed and where the
pages describe it.
"""
from .oracle import *  # noqa: F401,F403
