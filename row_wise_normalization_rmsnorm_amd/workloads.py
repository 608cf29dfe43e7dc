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
    op: str           # "rmsnorm", "add_rmsnorm", "add_rmsnorm_ag" or "block_sum"
    dtype: str        # "f32", "f16", "bf16" (block_sum also "fp8_e4m3", "fp8_e5m2", "i8")
    rows: int
    hidden: int
    k: int            # partial buffers (0 for plain RMSNorm)
    eps: float
    part_std: float   # std of x / each partial
    special_frac: float = 0.0  # fraction of rows scaled by 1e3, and (disjoint) all-zero
    seed: int = 0
    gather: int = 0   # add_rmsnorm_ag: output buffers that each receive the rows

    @property
    def fused(self) -> bool:
        return self.op in ("add_rmsnorm", "add_rmsnorm_ag")

    @property
    def itemsize(self) -> int:
        return {"f32": 4, "f16": 2, "bf16": 2}.get(self.dtype, 1)

    def algorithmic_bytes(self) -> int:
        """Bytes a single pass must move: each tensor element read or written
        once, gamma counted once.  Plain: read x, write out.  Fused: read K
        partials and the residual, write the residual and out (with the
        all-gather epilogue, every one of the gather outputs).  Block sum:
        read x, write one 4-byte result."""
        n = self.rows * self.hidden * self.itemsize
        if self.op == "block_sum":
            return n + 4
        per_elem = 2 if not self.fused else self.k + 2 + max(1, self.gather)
        return n * per_elem + self.hidden * self.itemsize

    def describe(self) -> str:
        if self.op == "block_sum":
            return f"block_sum {self.dtype} {self.rows}x{self.hidden}"
        return (f"{self.op} {self.dtype} rows={self.rows} hidden={self.hidden}"
                + (f" K={self.k}" if self.fused else "")
                + (f" outputs={self.gather}" if self.gather else "") + f" eps={self.eps:g}")


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
    # One rank's share of the K = 8 workload over 8 ranks with the all-gather
    # epilogue: 4096 / 8 rows reduced over the 8 ranks' partials, normalised,
    # and stored into the 8 ranks' gather buffers.
    "add_rmsnorm_ag_bf16_512x8192_k8_w8": Workload(
        "add_rmsnorm_ag_bf16_512x8192_k8_w8", "add_rmsnorm_ag", "bf16", 512, 8192, 8, 1e-5,
        0.125 ** 0.5, gather=8),
}

# Block all-reduce sum of a [S, K] tensor (page "Block All Reduce CUDA代码学习":
# S = K = 1024 randn, and K = 4096), every input dtype, plus a large bf16
# tensor for bandwidth.
for _dt in ("f32", "f16", "bf16", "fp8_e4m3", "fp8_e5m2", "i8"):
    WORKLOADS[f"block_sum_{_dt}_1024x1024"] = Workload(
        f"block_sum_{_dt}_1024x1024", "block_sum", _dt, 1024, 1024, 0, 0.0, 1.0)
WORKLOADS["block_sum_f32_4096x4096"] = Workload(
    "block_sum_f32_4096x4096", "block_sum", "f32", 4096, 4096, 0, 0.0, 1.0)
WORKLOADS["block_sum_bf16_16384x16384"] = Workload(
    "block_sum_bf16_16384x16384", "block_sum", "bf16", 16384, 16384, 0, 0.0, 1.0)

RMSNORM_WORKLOADS = [n for n, w in WORKLOADS.items() if w.op != "block_sum"]
BLOCK_SUM_WORKLOADS = [n for n, w in WORKLOADS.items() if w.op == "block_sum"]

# The headline workload: fused residual add + RMSNorm, bf16, 8192 x 4096.
HEADLINE = "add_rmsnorm_bf16_8192x4096_k1"


# GEMM with a reduce-scatter epilogue (page "LLM System: 通信计算融合算子实现
# 01 - sm80GEMM + ReduceScatter": the FFN's second GEMM, whose output is
# reduce-scattered over the tensor-parallel ranks).  One rank's share: tokens
# m, hidden n, and the rank's slice k of the FFN's intermediate dimension.
@dataclass(frozen=True)
class GemmWorkload:
    name: str
    dtype: str        # "bf16" or "f16"
    m: int            # tokens (rows of A and of the output)
    n: int            # hidden size (rows of the weight B)
    k: int            # intermediate slice (columns of A and B)
    world: int        # ranks: the output's rows split into this many chunks
    rank: int = 0
    alpha: float = 1.0
    beta: float = 0.0
    with_c: bool = False
    seed: int = 0
    op = "gemm_scatter"

    @property
    def a_std(self) -> float:
        return 1.0

    @property
    def b_std(self) -> float:
        """Weights scaled so each rank's partial output is N(0, 1/8), the
        partials' distribution of the K = 8 fused normalisation."""
        return (8.0 * self.k) ** -0.5

    def flops(self) -> int:
        return 2 * self.m * self.n * self.k

    def algorithmic_bytes(self) -> int:
        """A, B (and C) read once, the output written once."""
        return 2 * (self.m * self.k + self.n * self.k + self.m * self.n * (2 if self.with_c else 1))

    def describe(self) -> str:
        return (f"gemm_scatter {self.dtype} m={self.m} n={self.n} k={self.k} world={self.world} "
                f"rank={self.rank}" + (" +C" if self.with_c else ""))


GEMM_WORKLOADS = {
    # Producer of the K = 8 workload's partials: 4096 tokens, hidden 8192, an
    # FFN intermediate of 28672 split over 8 ranks (3584 per rank).
    "gemm_scatter_bf16_4096x8192x3584_w8": GemmWorkload(
        "gemm_scatter_bf16_4096x8192x3584_w8", "bf16", 4096, 8192, 3584, 8),
    "gemm_scatter_f16_4096x8192x3584_w8": GemmWorkload(
        "gemm_scatter_f16_4096x8192x3584_w8", "f16", 4096, 8192, 3584, 8),
    # The same layer at 1024 tokens: 128 tiles of 256 x 256 would leave half
    # of the 256 CUs idle, so this size takes the 128-wide tiles.
    "gemm_scatter_bf16_1024x8192x3584_w8": GemmWorkload(
        "gemm_scatter_bf16_1024x8192x3584_w8", "bf16", 1024, 8192, 3584, 8),
}
GEMM_HEADLINE = "gemm_scatter_bf16_4096x8192x3584_w8"
