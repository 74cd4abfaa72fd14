"""Reduced Matrix Multiplication (RMM) hot path for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI declared in
include/rmm.h (librmm.so, built in-tree); this package is the thin Python
binding with the same entry-point names.  There is no CPU fallback: calls
raise if the library is not built or no HIP device is present.
"""
from .binding import *  # noqa: F401,F403
from .binding import __all__  # noqa: F401
