"""Launches with the split_k that lowm_pick_split_k chooses, on the GPU,
judged against the fp64 oracle.  The choice is a table of the split_k
measured fastest per shape (bench.py --split-sweep); any split_k is correct,
and these tests check that the chosen one runs and gives the product: at grid
points of the table and at shapes between them (M 1 .. 64, N 768 .. 24576,
K 2048 .. 16384).  Large shapes are judged on sampled column windows (the
first 64 columns, a middle window and the ragged end), which the oracle
computes column by column; bf16 output must equal RNE of the fp32 sibling."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import split_bf16_gemm_amd as sbg
import workloads
from checks import assert_bf16, assert_fp32
from gpu_util import device, inputs, report, say, to_bits

pytestmark = pytest.mark.gpu

SHAPES = [  # grid points, then shapes between them
    (4, 768, 4096), (4, 6144, 4096), (4, 24576, 16384), (16, 1536, 8192), (1, 3072, 2048),
    (8, 12288, 8192), (2, 1000, 3072), (12, 5000, 12288), (16, 20000, 2048), (5, 2304, 12288),
    (32, 6144, 4096), (64, 3000, 8192),
]


def windows(N):
    w = min(64, N)
    mid = (N // 2) // 16 * 16
    out = [(0, w), (mid, min(N, mid + 64)), (max(0, N - 37), N)]
    return sorted(set(out))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_picked_split_k_against_the_oracle(M, N, K):
    lib = sbg.load()
    dev = device()
    S = lib.pick_split_k(M, N, K)
    assert S in (1, 2, 4, 8) and K % (8 * S) == 0
    wl = workloads.Workload(f"pick_{M}_{N}_{K}", M, N, K, S, seed_a=500 + M, seed_w=600 + N)
    A, W = inputs(wl)
    Ad, Wd = A.to(dev), W.to(dev)
    say("picked split_k", M, N, K, S)
    ws = lib.make_workspace(M, N, K, S, dev)
    c32 = lib.gemm(Ad, Wd, S, workspace=ws, out_dtype=torch.float32)
    c16 = lib.gemm(Ad, Wd, S, workspace=ws)
    torch.cuda.synchronize()
    c32, b16 = c32.cpu().numpy(), to_bits(c16)
    assert np.array_equal(b16, oracle.round_bf16(c32.astype(np.float64)))
    a_bits, w_bits = workloads.bits(A), workloads.bits(W)
    for n0, n1 in windows(N):
        C, Sc = oracle.gemm_cols(a_bits, w_bits, n0, n1)
        what = f"pick {M}x{N}x{K} split_k {S} cols {n0}:{n1}"
        assert_fp32(c32[:, n0:n1], C, Sc, what=what)
        report(what, assert_bf16(b16[:, n0:n1], C, Sc, K, oracle.default(), c32[:, n0:n1],
                                 what=what), C.size)
    if ws is not None:
        assert not ws.cpu().numpy().any()
