"""Synthetic workloads shaped like the paper's propagation configurations.

Grids are ViT patch-14 token grids (378 px -> 27, 1036 px -> 74,
2072 px -> 148) with the compressed latent width C_c = 64 (C = 1152
compressed by s = 18), plus a tiny case and an uncompressed wide case.
Every tensor is drawn N(0, 1) by `inputs` (then rounded to the storage type).
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    C: int
    H: int
    W: int
    dtype: str          # storage type of every tensor; arithmetic is fp32
    seeds: tuple

    @property
    def pixels(self) -> int:
        return self.B * self.C * self.H * self.W

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes the operator must move: read x, lambda, u and 4 x 3 taps, write y."""
        return 16 * self.elem_bytes * self.pixels


WORKLOADS = {
    "tiny": Workload("tiny", 1, 8, 16, 16, "fp32", (0, 1, 2, 3, 4)),
    "base378": Workload("base378", 8, 64, 27, 27, "fp32", (0, 1)),
    "latent1k": Workload("latent1k", 32, 64, 74, 74, "bf16", (0, 1)),
    "wide256": Workload("wide256", 1, 1024, 256, 256, "fp32", (0,)),
    "latent2k": Workload("latent2k", 4, 64, 148, 148, "bf16", (0,)),
}

# The workload the throughput metric is quoted on.
METRIC_WORKLOAD = "latent1k"
