"""Batched launches: several independent GEMMs that share M, K and split_k in
one kernel launch.  Each GEMM of a batch must equal, bit for bit, the single
launch of the same product (same kernel, same summation order); the first one
is also judged against the oracle, and the whole workspace (counters and
partial slots) must be zero again afterwards."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import split_bf16_gemm_amd as sbg
import workloads
from gpu_util import assert_bf16_launch, device, inputs, say, to_bits

pytestmark = pytest.mark.gpu

CASES = [
    (4, [6144, 1024, 1024], 4096, 2),      # a wide projection and two narrow ones
    (4, [300, 17, 2304, 64], 2048, 4),     # ragged N
    (20, [512, 640, 96], 2048, 2),         # two activation blocks
    (4, [1024, 2048], 1024, 1),            # split_k 1: no workspace
    (1, [6144] * 8, 4096, 8),              # the largest batch
    (4, [768], 4096, 2),                   # a batch of one
    (8, [6144, 6144], 4096, 1),            # quarter tiles of 32 rows for every GEMM
    (8, [6144, 1024], 4096, 1),            # quarter tiles, one width for every N
    (24, [6144, 512], 4096, 2),            # quarter tiles: 16 rows for the batch, 64 alone
    (64, [6144, 1024], 4096, 1),           # quarter tiles: 16 rows for the batch, 32 alone
    (64, [2048, 6144], 4096, 1),           # quarter-rows tiles: 16 columns for the batch, 48 alone
    (56, [12288, 1000], 2048, 1),          # quarter-rows for the batch, 64-row quarter tiles alone
]


def batch_workloads(M, Ns, K, S):
    return [workloads.Workload(f"batch_m{M}_n{N}_k{K}_s{S}_{g}", M, N, K, S,
                               seed_a=100 + g, seed_w=200 + g)
            for g, N in enumerate(Ns)]


@pytest.mark.parametrize("M,Ns,K,S", CASES)
def test_batch_equals_single_launches(M, Ns, K, S):
    lib = sbg.load()
    dev = device()
    wls = batch_workloads(M, Ns, K, S)
    As = [inputs(wl)[0].to(dev) for wl in wls]
    Ws = [inputs(wl)[1].to(dev) for wl in wls]
    ws = None
    if S > 1:
        ws = torch.zeros(lib.batched_workspace_bytes(M, Ns, K, S), dtype=torch.uint8,
                         device=dev)
    say("batched", M, Ns, K, S)
    outs = lib.gemm_batched(As, Ws, S, workspace=ws)
    torch.cuda.synchronize()
    got = [to_bits(o) for o in outs]
    for g, wl in enumerate(wls):
        single = lib.gemm(As[g], Ws[g], S, workspace=lib.make_workspace(M, Ns[g], K, S, dev))
        torch.cuda.synchronize()
        assert np.array_equal(got[g], to_bits(single)), \
            f"GEMM {g} of the batch differs from its single launch"
    assert_bf16_launch(lib, As[0], Ws[0], wls[0], got[0], what="batch GEMM 0")
    if ws is not None:
        assert not ws.cpu().numpy().any(), "a counter or partial slot of the batch was left non-zero"


def test_batch_reuses_its_workspace():
    """Two batches in a row on one workspace, the second with other shapes."""
    lib = sbg.load()
    dev = device()
    K, S = 2048, 2
    first = batch_workloads(4, [2304, 512], K, S)
    second = batch_workloads(4, [96, 33, 640], K, S)
    size = max(lib.batched_workspace_bytes(4, [w.N for w in first], K, S),
               lib.batched_workspace_bytes(4, [w.N for w in second], K, S))
    ws = torch.zeros(size, dtype=torch.uint8, device=dev)
    for wls in (first, second):
        As = [inputs(wl)[0].to(dev) for wl in wls]
        Ws = [inputs(wl)[1].to(dev) for wl in wls]
        say("batched reuse", [w.N for w in wls])
        outs = lib.gemm_batched(As, Ws, S, workspace=ws)
        torch.cuda.synchronize()
        for g, wl in enumerate(wls):
            single = lib.gemm(As[g], Ws[g], S, workspace=lib.make_workspace(4, wl.N, K, S, dev))
            torch.cuda.synchronize()
            assert np.array_equal(to_bits(outs[g]), to_bits(single))


@pytest.mark.parametrize("S", [1, 2])
def test_batch_may_share_one_activation(S):
    """Projections of one activation (query, key and value weights): every
    GEMM of the batch reads the same A, which the launch allows since inputs
    are only read."""
    lib = sbg.load()
    dev = device()
    M, K, Ns = 4, 4096, [6144, 1024, 1024]
    wls = batch_workloads(M, Ns, K, S)
    A = inputs(wls[0])[0].to(dev)
    Ws = [inputs(wl)[1].to(dev) for wl in wls]
    ws = None
    if S > 1:
        ws = torch.zeros(lib.batched_workspace_bytes(M, Ns, K, S), dtype=torch.uint8,
                         device=dev)
    say("batched shared A", M, Ns, K, S)
    outs = lib.gemm_batched([A] * len(Ws), Ws, S, workspace=ws)
    torch.cuda.synchronize()
    for g, wl in enumerate(wls):
        single = lib.gemm(A, Ws[g], S, workspace=lib.make_workspace(M, Ns[g], K, S, dev))
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(outs[g]), to_bits(single)), \
            f"GEMM {g} over the shared activation differs from its single launch"
    assert_bf16_launch(lib, A, Ws[0], wls[0], to_bits(outs[0]), what="shared-A GEMM 0")
    if ws is not None:
        assert not ws.cpu().numpy().any(), "the shared-A batch left its workspace non-zero"


def test_overlapping_outputs_are_refused_before_any_kernel():
    """Two outputs of one batch on the same memory: the launch returns an
    invalid-argument error and leaves every buffer as it was."""
    lib = sbg.load()
    dev = device()
    M, K, S, N = 4, 1024, 2, 512
    wls = batch_workloads(M, [N, N], K, S)
    As = [inputs(wl)[0].to(dev) for wl in wls]
    Ws = [inputs(wl)[1].to(dev) for wl in wls]
    shared = torch.full((M, N), 1.5, dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(lib.batched_workspace_bytes(M, [N, N], K, S), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    say("batched overlapping outputs", M, N, K, S)
    with pytest.raises(sbg.binding.LowmError, match="overlap"):
        lib.gemm_batched(As, Ws, S, outs=[shared, shared], workspace=ws)
    torch.cuda.synchronize()
    assert bool((shared == 1.5).all()), "a refused launch wrote its output"
    assert not ws.cpu().numpy().any(), "a refused launch touched the workspace"
