"""Seeded synthetic inputs for the FP16 GEMM workloads.

This module is shared by the tests, the smoke check and the benchmark, and
serves both the GPU library and the CPU oracle.  It holds none of the GEMM's
arithmetic: it only draws operand matrices and the sampled row / column
index sets.

Recipe (one ``torch.Generator('cpu')`` per workload, seeded with the
workload's seed; A (M x K) is drawn first, then B (K x N), in float32, then
rounded to binary16 by ``.to(torch.float16)``):

* ``uniform``   -- A, B ~ U[-1, 1): ``2 * rand - 1``.
* ``normal``    -- A, B ~ N(0, sigma = 1/sqrt(K)): ``randn / sqrt(K)``.
* ``mlp``       -- activations A ~ N(0, 1), weights B ~ N(0, 1/sqrt(K)).

The pages benchmark FP16 GEMM at unstated sizes; these five shapes (plus the
one-GPU shard of the largest, 8192 x 3584 x 8192) stand in for them.  For the largest shapes the
oracle checks a 4096 x 4096 block at seeded random rows R and columns S:
``randperm(M)[:4096]`` then ``randperm(N)[:4096]`` from a generator seeded
with ``seed + 1000``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str        # "uniform" | "normal" | "mlp"
    seed: int
    relu: bool = False
    sampled: bool = False   # oracle checks a 4096 x 4096 seeded block instead of all of C

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def min_bytes(self) -> int:
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N)


WORKLOADS = {
    "gemm_256": Workload("gemm_256", 256, 256, 256, "uniform", 0),
    "gemm_1024_relu": Workload("gemm_1024_relu", 1024, 1024, 1024, "uniform", 1, relu=True),
    "gemm_4096": Workload("gemm_4096", 4096, 4096, 4096, "normal", 2),
    "gemm_ragged_3000x5000x4100": Workload("gemm_ragged_3000x5000x4100", 3000, 5000, 4100, "uniform", 3),
    "gemm_8192": Workload("gemm_8192", 8192, 8192, 8192, "mlp", 4, sampled=True),
    "gemm_mlp_8192x28672x8192": Workload("gemm_mlp_8192x28672x8192", 8192, 28672, 8192, "mlp", 4,
                                         sampled=True),
    # one GPU's column block of the MLP projection when it is split over 8 GPUs along N
    "gemm_mlp_shard_8192x3584x8192": Workload("gemm_mlp_shard_8192x3584x8192", 8192, 3584, 8192, "mlp", 4,
                                              sampled=True),
}

SAMPLE = 4096


def make_inputs(w: Workload) -> tuple[torch.Tensor, torch.Tensor]:
    """Draw (A, B) as contiguous CPU float16 tensors for workload ``w``."""
    return draw(w.M, w.N, w.K, w.dist, w.seed)


def draw(M: int, N: int, K: int, dist: str, seed: int) -> tuple[torch.Tensor, torch.Tensor]:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    if dist == "uniform":
        a = torch.rand((M, K), generator=g, dtype=torch.float32) * 2.0 - 1.0
        b = torch.rand((K, N), generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal":
        s = 1.0 / math.sqrt(K) if K > 0 else 1.0
        a = torch.randn((M, K), generator=g, dtype=torch.float32) * s
        b = torch.randn((K, N), generator=g, dtype=torch.float32) * s
    elif dist == "mlp":
        s = 1.0 / math.sqrt(K) if K > 0 else 1.0
        a = torch.randn((M, K), generator=g, dtype=torch.float32)
        b = torch.randn((K, N), generator=g, dtype=torch.float32) * s
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return a.to(torch.float16).contiguous(), b.to(torch.float16).contiguous()


def draw_ints(M: int, N: int, K: int, seed: int, lo: int = -2, hi: int = 2):
    """Integer-valued binary16 operands in [lo, hi]: every fp32 partial sum of
    their products is an integer below 2^24, so any accumulation order gives
    the exact integer product."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    a = torch.randint(lo, hi + 1, (M, K), generator=g, dtype=torch.int64)
    b = torch.randint(lo, hi + 1, (K, N), generator=g, dtype=torch.int64)
    return a.to(torch.float16).contiguous(), b.to(torch.float16).contiguous()


def sample_indices(w: Workload, n: int = SAMPLE) -> tuple[torch.Tensor, torch.Tensor]:
    """Seeded rows R (from [0, M)) and columns S (from [0, N)) for the sampled check."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 1000)
    rows = torch.randperm(w.M, generator=g)[: min(n, w.M)]
    cols = torch.randperm(w.N, generator=g)[: min(n, w.N)]
    return rows, cols


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()
