"""Seeded synthetic workloads for the low-M split-K bf16 GEMM.

This module only draws inputs.  It holds none of the product's arithmetic and
is the one piece both the oracle side and the HIP side use.

Shapes and value distributions follow the pages:
  * the integer closed form of the Triton issue "warpgroup_mma_wait does not
    properly synchronize across warpgroups" (Describe the bug): an all-ones
    operand times integers drawn uniformly from [-3, 3] with seed 0, so every
    partial sum is an integer far below 2^24 and exact in fp32;
  * the three shapes of the TensorRT-LLM PR "Fix two synchronization gaps in
    the MiniMax M3 low-M split-K GEMM" (Hardware verification): M 4 with
    N 6144 / K 4096 / split_k 2, N 2304 / K 12288 / split_k 4, and N 49152.
The random-valued cases draw A ~ N(0, 1) and W ~ N(0, 0.02) (0.02 read as the
standard deviation) in fp32 and cast to bf16 with torch's round-to-nearest-even.
They stand in for the activations and weights of the model the PR serves,
which are neither needed nor available.
"""
from __future__ import annotations

import re

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    split_k: int
    kind: str = "randn"          # "randn" | "int_closed_form" | "int_both"
    seed_a: int = 0
    seed_w: int = 0
    tags: tuple = field(default=())

    def describe(self) -> dict:
        return {"workload": self.name, "M": self.M, "N": self.N, "K": self.K,
                "split_k": self.split_k, "inputs": self.kind,
                "seed_a": self.seed_a, "seed_w": self.seed_w}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def make_inputs(wl: Workload):
    """(A, W) as contiguous CPU bf16 tensors of shapes [M, K] and [N, K]."""
    M, N, K = wl.M, wl.N, wl.K
    if wl.kind == "int_closed_form":
        A = torch.ones((M, K), dtype=torch.bfloat16)
        W = torch.randint(-3, 4, (N, K), generator=_gen(wl.seed_w),
                          dtype=torch.int64).to(torch.bfloat16)
    elif wl.kind == "int_both":
        A = torch.randint(-3, 4, (M, K), generator=_gen(wl.seed_a),
                          dtype=torch.int64).to(torch.bfloat16)
        W = torch.randint(-3, 4, (N, K), generator=_gen(wl.seed_w),
                          dtype=torch.int64).to(torch.bfloat16)
    elif wl.kind == "randn":
        A = torch.randn((M, K), generator=_gen(wl.seed_a),
                        dtype=torch.float32).to(torch.bfloat16)
        W = (torch.randn((N, K), generator=_gen(wl.seed_w), dtype=torch.float32)
             * 0.02).to(torch.bfloat16)
    else:
        raise ValueError(f"unknown input kind {wl.kind!r}")
    return A.contiguous(), W.contiguous()


def make_large_w(N: int, K: int, seed: int, device) -> torch.Tensor:
    """W [N, K] drawn on `device` for operands too large to draw on the host:
    N(0, 0.02) in fp32 from a seeded torch generator on that device, cast to
    bf16 with round-to-nearest-even, 8192 rows at a time.  The values differ
    from a host draw of the same seed; a test copies the rows it judges back
    to the host for the oracle."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    W = torch.empty((N, K), dtype=torch.bfloat16, device=device)
    for r0 in range(0, N, 8192):
        r1 = min(N, r0 + 8192)
        W[r0:r1] = (torch.randn((r1 - r0, K), generator=g, device=device,
                                dtype=torch.float32) * 0.02).to(torch.bfloat16)
    return W


def bits(t: torch.Tensor):
    """The uint16 bit patterns of a CPU bf16 tensor, as a numpy array."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# The integer closed form (Triton issue, Describe the bug), at the size the
# oracle finishes in well under a second.
INT_EXACT = Workload("int_closed_form_m4_n512_k1024_s2", 4, 512, 1024, 2,
                     kind="int_closed_form", seed_a=0, seed_w=0)

# The three shapes of the PR's Hardware verification.
HEADLINE = Workload("m4_n6144_k4096_s2", 4, 6144, 4096, 2,
                    seed_a=1001, seed_w=2001)
SPLITK4 = Workload("m4_n2304_k12288_s4", 4, 2304, 12288, 4,
                   seed_a=1002, seed_w=2002)
WIDE_N = Workload("m4_n49152_k4096_s2", 4, 49152, 4096, 2,
                  seed_a=1003, seed_w=2003)

SWEEP_M = (1, 8, 16, 32, 64)
SWEEP_S = (1, 2, 4, 8)


def sweep():
    """M in {1, 8, 16, 32, 64} x split_k in {1, 2, 4, 8} at N 6144, K 4096."""
    out = []
    for i, m in enumerate(SWEEP_M):
        for j, s in enumerate(SWEEP_S):
            out.append(Workload(f"sweep_m{m}_n6144_k4096_s{s}", m, 6144, 4096, s,
                                seed_a=1100 + 10 * i + j,
                                seed_w=2100 + 10 * i + j))
    return out


ALL = [INT_EXACT, HEADLINE, SPLITK4, WIDE_N] + sweep()


def by_name(name: str) -> Workload:
    """A named workload, or any shape written mM_nN_kK_sS (seeded from its
    sizes, the distributions of the random workloads)."""
    for wl in ALL:
        if wl.name == name:
            return wl
    m = re.fullmatch(r"m(\d+)_n(\d+)_k(\d+)_s(\d+)", name)
    if m:
        M, N, K, S = (int(x) for x in m.groups())
        return Workload(name, M, N, K, S, seed_a=3000 + M, seed_w=4000 + N % 997 + K % 991 + S)
    raise KeyError(name)
