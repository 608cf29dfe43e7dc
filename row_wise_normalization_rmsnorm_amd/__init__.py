"""Row-wise RMSNorm and fused K-partial + residual + RMSNorm for MI355X (gfx950).

The compute path is ``librmsnorm.so``: hand-written HIP kernels behind a C ABI
(``include/rmsnorm.h``).  The Python layer only marshals torch tensors into
pointers and the current HIP stream.  Nothing here falls back to CPU or torch
arithmetic: if the library is missing, calls raise.
"""
from .workloads import WORKLOADS, HEADLINE, Workload  # noqa: F401

__all__ = ["WORKLOADS", "HEADLINE", "Workload"]
