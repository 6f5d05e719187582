"""Launches captured in a HIP graph and replayed (launch-latency hiding for a
caller that replays a fixed sequence of GEMMs).  The launch path writes no
memory outside its kernels: the workspace goes back to zero inside the kernel,
with no memset, so a captured launch replays like an eager one.  Every replay
must equal the eager launch bit for bit and leave the workspace zero, with
eager launches on the same workspace between the replays; the eager result is
judged against the oracle as in the parity tests."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import split_bf16_gemm_amd as sbg
import workloads
from gpu_util import assert_bf16_launch, device, inputs, say, to_bits

pytestmark = pytest.mark.gpu

REPLAYS = 3
LAUNCHES_PER_GRAPH = 3

CASES = [
    (4, 6144, 4096, 2),     # line-pair tiles, the tile's last rank folds early
    (4, 2304, 12288, 4),    # line-pair tiles, split_k 4
    (1, 6144, 4096, 8),     # line-pair tiles on the counter path
    (16, 1000, 2048, 2),    # quarter tiles, strip epilogue, ragged N
    (64, 520, 2048, 2),     # panel tiles, ragged N
    (16, 6144, 4096, 1),    # quarter tiles without split-K: no workspace
    (64, 4096, 4096, 1),    # quarter-rows tiles: two row blocks per tile
]


def _check_workspace(lib, ws, N, what):
    if ws is None:
        return
    assert lib.workspace_status(ws, N) == (0, 0), f"{what}: counter words left set"
    assert not ws.cpu().numpy().any(), f"{what}: workspace not zero after the launch"


@pytest.mark.parametrize("M,N,K,S", CASES)
def test_graph_replays_equal_the_eager_launch(M, N, K, S):
    lib = sbg.load()
    dev = device()
    wl = workloads.Workload(f"graph_m{M}_n{N}_k{K}_s{S}", M, N, K, S,
                            seed_a=700 + M, seed_w=800 + S)
    A_cpu, W_cpu = inputs(wl)
    A, W = A_cpu.to(dev), W_cpu.to(dev)
    ws = lib.make_workspace(M, N, K, S, dev)
    eager = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    say("graph eager", M, N, K, S)
    lib.gemm(A, W, S, out=eager, workspace=ws)
    torch.cuda.synchronize()
    ref = to_bits(eager)
    assert_bf16_launch(lib, A, W, wl, ref, what=f"graph eager {wl.name}")
    _check_workspace(lib, ws, N, "eager")

    outs = [torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
            for _ in range(LAUNCHES_PER_GRAPH)]
    s = torch.cuda.Stream(device=dev)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    say("graph capture", M, N, K, S)
    with torch.cuda.graph(g, stream=s):
        for o in outs:
            lib.gemm(A, W, S, out=o, workspace=ws)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for o in outs:
            o.zero_()
        say("graph replay", r, M, N, K, S)
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(to_bits(o), ref), f"replay {r}, launch {i} differs from eager"
        _check_workspace(lib, ws, N, f"replay {r}")
        # an eager launch on the same workspace between replays
        again = lib.gemm(A, W, S, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(again), ref), f"eager launch after replay {r} differs"
        _check_workspace(lib, ws, N, f"eager after replay {r}")


def test_graph_replays_a_batched_launch():
    """A batched launch (three GEMMs, one launch) captured once and replayed."""
    lib = sbg.load()
    dev = device()
    M, K, S = 4, 4096, 2
    Ns = [6144, 1024, 1024]
    wls = [workloads.Workload(f"graph_batch_m{M}_n{N}_k{K}_s{S}_{i}", M, N, K, S,
                              seed_a=900 + i, seed_w=950 + i) for i, N in enumerate(Ns)]
    As = [inputs(wl)[0].to(dev) for wl in wls]
    Ws = [inputs(wl)[1].to(dev) for wl in wls]
    ws = torch.zeros(lib.batched_workspace_bytes(M, Ns, K, S), dtype=torch.uint8, device=dev)
    say("graph batched eager", Ns)
    ref = [to_bits(o) for o in lib.gemm_batched(As, Ws, S, workspace=ws)]
    torch.cuda.synchronize()
    assert_bf16_launch(lib, As[0], Ws[0], wls[0], ref[0], what="graph batched GEMM 0")
    outs = [torch.zeros((M, N), dtype=torch.bfloat16, device=dev) for N in Ns]
    s = torch.cuda.Stream(device=dev)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        lib.gemm_batched(As, Ws, S, outs=outs, workspace=ws)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for o in outs:
            o.zero_()
        say("graph batched replay", r)
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(to_bits(o), ref[i]), f"replay {r}, GEMM {i} differs"
        assert not ws.cpu().numpy().any(), f"replay {r} left the batch workspace non-zero"
