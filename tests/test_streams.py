"""Launches in flight at once on different streams, each with its own
workspace.  Nothing but the workspace is shared state of a launch, so
concurrent launches of different shapes and tile families must each give
the bits of the same launch run alone, and leave their workspaces zero."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import split_bf16_gemm_amd as sbg
import workloads
from gpu_util import assert_bf16_launch, device, inputs, say, to_bits

pytestmark = pytest.mark.gpu

ROUNDS = 8

PAIRS = [
    # line-pair tiles with the early owner beside quarter tiles on the counter path
    ((4, 6144, 4096, 2), (16, 2304, 4096, 4)),
    # panel tiles beside line-pair tiles on the counter path
    ((64, 1040, 2048, 2), (1, 3072, 4096, 8)),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_concurrent_streams_give_the_bits_of_a_lone_launch(first, second):
    lib = sbg.load()
    dev = device()
    wls = [workloads.Workload(f"streams_m{M}_n{N}_k{K}_s{S}", M, N, K, S,
                              seed_a=600 + M, seed_w=650 + S)
           for (M, N, K, S) in (first, second)]
    ops = [tuple(t.to(dev) for t in inputs(wl)) for wl in wls]
    wss = [lib.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev) for wl in wls]
    alone = []
    for wl, (A, W), ws in zip(wls, ops, wss):
        say("streams alone", wl.name)
        alone.append(to_bits(lib.gemm(A, W, wl.split_k, workspace=ws)))
        torch.cuda.synchronize()
        assert_bf16_launch(lib, A, W, wl, alone[-1], what=f"alone {wl.name}")
    streams = [torch.cuda.Stream(device=dev) for _ in wls]
    outs = [[torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev)
             for _ in range(ROUNDS)] for wl in wls]
    torch.cuda.synchronize()
    say("streams concurrent", [wl.name for wl in wls])
    for r in range(ROUNDS):
        for i, (wl, (A, W), ws, s) in enumerate(zip(wls, ops, wss, streams)):
            lib.gemm(A, W, wl.split_k, out=outs[i][r], workspace=ws, stream=s)
    torch.cuda.synchronize()
    for i, wl in enumerate(wls):
        for r in range(ROUNDS):
            assert np.array_equal(to_bits(outs[i][r]), alone[i]), \
                f"{wl.name}, launch {r} beside the other stream differs from a lone launch"
        if wss[i] is not None:
            assert not wss[i].cpu().numpy().any(), f"{wl.name} left its workspace non-zero"
