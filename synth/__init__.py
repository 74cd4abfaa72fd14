"""Seeded synthetic inputs for the RMM hot path.

This package only *draws* operands (activations, weights, Q/K/V, attention
probabilities) with the shapes and value distributions of the workloads the
pages evaluate on.  It contains none of the reduction method's arithmetic (no
column scores, no selection, no reduced product), so it can feed both the CPU
oracle and the HIP library without coupling them.
"""
from .gen import *  # noqa: F401,F403
from .workloads import *  # noqa: F401,F403
