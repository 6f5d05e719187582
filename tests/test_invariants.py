"""Invariants of the product on the GPU that hold at any size and pin
position and operand mix-ups that the closed form of the Triton issue
"warpgroup_mma_wait does not properly synchronize across warpgroups"
(Describe the bug) cannot see, since it makes every row of C equal:

  * permuting the rows of W permutes the columns of C, bit for bit (each
    output element is summed in the same order wherever its column sits);
  * permuting the rows of A permutes the rows of C, bit for bit;
  * scaling A by 2 scales C by 2, bit for bit (exact in bf16 and fp32);
  * integer-valued inputs are linear, exactly: C(A, W1 + W2) = C(A, W1) +
    C(A, W2) and C(A1 + A2, W) = C(A1, W) + C(A2, W) (every partial sum is an
    integer far below 2^24).
Each runs for the default tactic of each tile family and for split_k 1 and
more."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import split_bf16_gemm_amd as sbg
import workloads
from gpu_util import device, inputs, say

pytestmark = pytest.mark.gpu

# (M, N, K, split_k): line-pair tiles with the early owner, panel tiles,
# the register ring (ragged K slice), quarter tiles of 32 rows without
# split-K, panel tiles with split_k 4, quarter tiles of 16 and of 64 rows
# with split_k 2.
SHAPES = [(4, 1000, 2048, 2), (40, 700, 1536, 3), (9, 333, 1032, 3), (16, 2048, 4096, 1),
          (64, 512, 4096, 4), (12, 1500, 2048, 2), (20, 3000, 2048, 2)]


def run32(lib, A, W, S, dev):
    out = lib.gemm(A, W, S, workspace=lib.make_workspace(A.shape[0], W.shape[0], A.shape[1], S,
                                                         dev), out_dtype=torch.float32)
    return out


def bits32(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("M,N,K,S", SHAPES)
def test_permuting_w_rows_permutes_c_columns(M, N, K, S):
    lib = sbg.load()
    dev = device()
    wl = workloads.Workload(f"perm_{M}_{N}", M, N, K, S, seed_a=M, seed_w=N)
    A, W = inputs(wl)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(N + K))
    Ad, Wd, Wp = A.to(dev), W.to(dev), W[perm].contiguous().to(dev)
    say("W-row permutation", M, N, K, S)
    c = run32(lib, Ad, Wd, S, dev)
    cp = run32(lib, Ad, Wp, S, dev)
    c16 = lib.gemm(Ad, Wd, S, workspace=lib.make_workspace(M, N, K, S, dev))
    cp16 = lib.gemm(Ad, Wp, S, workspace=lib.make_workspace(M, N, K, S, dev))
    torch.cuda.synchronize()
    assert np.array_equal(bits32(cp), bits32(c)[:, perm.numpy()])
    assert torch.equal(cp16.cpu().view(torch.int16), c16.cpu().view(torch.int16)[:, perm])


@pytest.mark.parametrize("M,N,K,S", SHAPES)
def test_permuting_a_rows_permutes_c_rows(M, N, K, S):
    lib = sbg.load()
    dev = device()
    wl = workloads.Workload(f"permA_{M}_{N}", M, N, K, S, seed_a=M + 1, seed_w=N + 1)
    A, W = inputs(wl)
    perm = torch.randperm(M, generator=torch.Generator().manual_seed(M + K))
    say("A-row permutation", M, N, K, S)
    c = run32(lib, A.to(dev), W.to(dev), S, dev)
    cp = run32(lib, A[perm].contiguous().to(dev), W.to(dev), S, dev)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(cp), bits32(c)[perm.numpy()])


@pytest.mark.parametrize("M,N,K,S", SHAPES)
def test_doubling_a_doubles_c(M, N, K, S):
    lib = sbg.load()
    dev = device()
    wl = workloads.Workload(f"scale_{M}_{N}", M, N, K, S, seed_a=M + 2, seed_w=N + 2)
    A, W = inputs(wl)
    say("doubling A", M, N, K, S)
    c = run32(lib, A.to(dev), W.to(dev), S, dev)
    c2 = run32(lib, (A * 2).to(dev), W.to(dev), S, dev)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(c2), bits32(c * 2))


@pytest.mark.parametrize("M,N,K,S", SHAPES)
def test_integer_inputs_are_linear(M, N, K, S):
    lib = sbg.load()
    dev = device()
    g = torch.Generator().manual_seed(M * N + K)
    ints = lambda r, c: torch.randint(-3, 4, (r, c), generator=g).to(torch.bfloat16)
    A1, A2, W1, W2 = ints(M, K), ints(M, K), ints(N, K), ints(N, K)
    say("integer linearity", M, N, K, S)
    d = lambda t: t.to(dev)
    cW = run32(lib, d(A1), d(W1 + W2), S, dev)     # |w| <= 6: exact in bf16
    cW1 = run32(lib, d(A1), d(W1), S, dev)
    cW2 = run32(lib, d(A1), d(W2), S, dev)
    cA = run32(lib, d(A1 + A2), d(W1), S, dev)
    cA2 = run32(lib, d(A2), d(W1), S, dev)
    torch.cuda.synchronize()
    assert float((cW.abs()).max()) < 2 ** 24
    assert torch.equal(cW.cpu(), (cW1 + cW2).cpu())
    assert torch.equal(cA.cpu(), (cW1 + cA2).cpu())
