"""The no-allocation entry point (lowm_gemm_splitk_noalloc): the same product
as lowm_gemm_splitk with the split-K workspace taken from the library's
built-in device scratch.  Each call is judged bit for bit against the
workspace entry point on the same inputs (same kernels and summation order),
and against the fp64 oracle, for pairs of calls in a row, the second one
smaller, so that the second call runs on the scratch the first one left."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import split_bf16_gemm_amd as sbg
import workloads
from gpu_util import assert_bf16_launch, device, inputs, say, to_bits

pytestmark = pytest.mark.gpu

PAIRS = [
    [(4, 6144, 4096, 2), (4, 512, 1024, 2)],        # line tiles, early owner
    [(64, 6144, 4096, 2), (20, 300, 2048, 4)],      # panel tiles, counter exchange
    [(16, 6144, 4096, 8), (3, 100, 1536, 3)],       # split_k 8, then a generic split_k
    [(4, 2304, 12288, 4), (1, 64, 512, 1)],         # split_k 4, then no workspace at all
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "->".join("x".join(map(str, c)) for c in p))
def test_noalloc_matches_the_workspace_entry_point(pair):
    lib = sbg.load()
    dev = device()
    for i, (M, N, K, S) in enumerate(pair):
        wl = workloads.Workload(f"noalloc_{M}_{N}_{K}_{S}", M, N, K, S, seed_a=300 + M, seed_w=400 + N)
        A, W = (t.to(dev) for t in inputs(wl))
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        say("noalloc call", i, M, N, K, S)
        lib.gemm_noalloc(A, W, S, out=out)
        ref = lib.gemm(A, W, S, workspace=lib.make_workspace(M, N, K, S, dev))
        torch.cuda.synchronize()
        got = to_bits(out)
        assert np.array_equal(got, to_bits(ref)), \
            f"call {i} ({M}x{N}x{K}, split_k {S}) differs from lowm_gemm_splitk"
        assert_bf16_launch(lib, A, W, wl, got, what=f"noalloc call {i}")


def test_noalloc_repeated_on_one_stream_then_another():
    """Back-to-back calls without synchronisation (each leaves the scratch
    clear for the next), then a call on a second stream after a sync."""
    lib = sbg.load()
    dev = device()
    wl = workloads.HEADLINE
    A, W = (t.to(dev) for t in inputs(wl))
    outs = [torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev) for _ in range(8)]
    say("noalloc back-to-back")
    for o in outs:
        lib.gemm_noalloc(A, W, wl.split_k, out=o)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=dev)
    last = torch.empty_like(outs[0])
    lib.gemm_noalloc(A, W, wl.split_k, out=last, stream=s)
    s.synchronize()
    ref = to_bits(lib.gemm(A, W, wl.split_k, workspace=lib.make_workspace(wl.M, wl.N, wl.K,
                                                                          wl.split_k, dev)))
    for o in outs + [last]:
        assert np.array_equal(to_bits(o), ref)
