"""CPU oracle for Reduced Matrix Multiplication (RMM).  TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy implementation of what the RMM hot path computes.
Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the product library never does, and it shares no
code with the HIP path.
"""
from .rmm_oracle import *  # noqa: F401,F403
