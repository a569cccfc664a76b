"""Seeded synthetic inputs shared by the oracle-side tests and the GPU-side tests/bench.

This package holds input generation only (random draws, their storage dtype and
layout).  It performs none of the FP8 method's arithmetic: no scaling, no FP8
encoding, no amax, no GEMM.  Both the CPU oracle and the HIP path receive the
same arrays from here; neither imports the other.
"""

from .workloads import *  # noqa: F401,F403
