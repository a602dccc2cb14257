"""Seeded synthetic inputs shared by the GPU path's harness and by the CPU oracle.

This package holds only input preparation: model shapes, seeded random draws,
bf16 rounding of the draws, block-table placement of synthetic cache contents.
It holds none of the decoder's arithmetic (norms, projections, rotary
embedding, attention, sampling) and imports neither the oracle nor the HIP
library.
"""
from .workloads import *  # noqa: F401,F403
