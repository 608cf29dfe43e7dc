"""The five synthetic workloads of the row-wise RMSNorm path.

Each names its call, dtype, shape, number of partials, eps and value
distribution.  Nothing here computes any part of the method.

The pages time RMSNorm on random data at shapes (512, 1592) and (512, 2048)
(page "RMSNorm kernel", section 2 "Performance" and section 3.1 "Vectorize")
and size the fused form per token with a residual and K rank partials (page
"Tokenweave fused-RMSNorm-AR kernel", "Code walkthrough").  The larger fused
shapes below are the hot path's production sizes; every input is seeded and
synthetic (no dataset is involved).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    op: str           # "rmsnorm" or "add_rmsnorm"
    dtype: str        # "f32", "f16" or "bf16"
    rows: int
    hidden: int
    k: int            # partial buffers (0 for plain RMSNorm)
    eps: float
    part_std: float   # std of x / each partial
    special_frac: float = 0.0  # fraction of rows scaled by 1e3, and (disjoint) all-zero
    seed: int = 0

    @property
    def fused(self) -> bool:
        return self.op == "add_rmsnorm"

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def algorithmic_bytes(self) -> int:
        """Bytes a single pass must move: each tensor element read or written
        once, gamma counted once.  Plain: read x, write out.  Fused: read K
        partials and the residual, write the residual and out."""
        n = self.rows * self.hidden * self.itemsize
        per_elem = 2 if not self.fused else self.k + 3
        return n * per_elem + self.hidden * self.itemsize

    def describe(self) -> str:
        return (f"{self.op} {self.dtype} rows={self.rows} hidden={self.hidden}"
                + (f" K={self.k}" if self.fused else "") + f" eps={self.eps:g}")


WORKLOADS = {
    "rmsnorm_f32_512x2048": Workload(
        "rmsnorm_f32_512x2048", "rmsnorm", "f32", 512, 2048, 0, 1e-6, 1.0),
    "rmsnorm_bf16_512x1592": Workload(
        "rmsnorm_bf16_512x1592", "rmsnorm", "bf16", 512, 1592, 0, 1e-6, 1.0),
    "rmsnorm_f16_512x1592": Workload(
        "rmsnorm_f16_512x1592", "rmsnorm", "f16", 512, 1592, 0, 1e-6, 1.0),
    "add_rmsnorm_bf16_8192x4096_k1": Workload(
        "add_rmsnorm_bf16_8192x4096_k1", "add_rmsnorm", "bf16", 8192, 4096, 1, 1e-6, 1.0),
    "add_rmsnorm_bf16_4096x8192_k8": Workload(
        "add_rmsnorm_bf16_4096x8192_k8", "add_rmsnorm", "bf16", 4096, 8192, 8, 1e-5,
        0.125 ** 0.5),
    "add_rmsnorm_bf16_65536x16384_k1": Workload(
        "add_rmsnorm_bf16_65536x16384_k1", "add_rmsnorm", "bf16", 65536, 16384, 1, 1e-6, 1.0,
        special_frac=0.01),
}

# The headline workload: fused residual add + RMSNorm, bf16, 8192 x 4096.
HEADLINE = "add_rmsnorm_bf16_8192x4096_k1"
