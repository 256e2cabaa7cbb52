"""Seeded synthetic inputs for the SharQ linear hot path.

This package holds input generation only -- random draws, the fp32 -> bf16
rounding of inputs, and MoE routing structure -- and none of the method's
arithmetic (no selection, no FP4 coding, no GEMM). Both the CPU oracle's tests
and the HIP path's tests and bench draw their inputs from here.
"""

from .workloads import *  # noqa: F401,F403
