"""Launch determinism of the split-K fold (headline shape, 20 launches).

The owner of a tile is whichever rank arrives last (or, where the last rank
finds every peer's partial already published, that rank), which varies from
launch to launch, but it always adds the partials in rank order, so the output
must not change in a single bit.  Following the PR "Fix two synchronization
gaps in the MiniMax M3 low-M split-K GEMM" (Hardware verification: 20 launches
per configuration, each compared bitwise with the unperturbed output), and so
that a race which reads a stale partial cannot hide behind identical inputs,
the launches alternate two input sets.  A partial slot holds the complement
of the fp32 bits, so a slot read before its rank wrote it decodes as NaN; and
every launch must leave the whole workspace (counters and partial slots) zero,
which the second run checks after each launch: a slot left uncleared
would hand the next launch's last rank a stale partial.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import split_bf16_gemm_amd as sbg
import workloads
from checks import assert_fp32
from gpu_util import assert_bf16_launch, device, inputs, oracle_result, say, to_bits

pytestmark = pytest.mark.gpu

LAUNCHES = 20


def two_sets(wl):
    other = workloads.Workload(wl.name + "_b", wl.M, wl.N, wl.K, wl.split_k,
                               seed_a=wl.seed_a + 500, seed_w=wl.seed_w + 500)
    return [wl, other]


@pytest.mark.parametrize("wl", [workloads.HEADLINE, workloads.SPLITK4,
                                workloads.by_name("sweep_m16_n6144_k4096_s8")],
                         ids=lambda w: w.name)
@pytest.mark.parametrize("check_ws", [False, True], ids=["back_to_back", "workspace_checked"])
def test_twenty_launches_bitwise(wl, check_ws):
    lib = sbg.load()
    dev = device()
    sets = two_sets(wl)
    ops = [tuple(t.to(dev) for t in inputs(s)) for s in sets]
    ws = lib.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    outs = [torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev) for _ in range(LAUNCHES)]
    say("determinism", wl.name, "workspace checked" if check_ws else "back-to-back")
    for i in range(LAUNCHES):
        A, W = ops[i % 2]
        lib.gemm(A, W, wl.split_k, out=outs[i], workspace=ws)
        if check_ws:
            torch.cuda.synchronize()
            assert int(ws.count_nonzero()) == 0, f"launch {i} left the workspace non-zero"
    torch.cuda.synchronize()
    bits = [to_bits(o) for o in outs]
    for i in range(2, LAUNCHES):
        assert np.array_equal(bits[i], bits[i % 2]), f"launch {i} differs from launch {i % 2}"
    assert not np.array_equal(bits[0], bits[1])
    for j, s in enumerate(sets):
        assert_bf16_launch(lib, *ops[j], s, bits[j], what=f"{s.name} launch {j}")
    assert not ws.cpu().numpy().any(), "the workspace was left non-zero"


def test_fp32_output_is_deterministic_too():
    lib = sbg.load()
    dev = device()
    wl = workloads.HEADLINE
    A, W = (t.to(dev) for t in inputs(wl))
    ws = lib.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    say("fp32 determinism")
    outs = [lib.gemm(A, W, wl.split_k, workspace=ws, out_dtype=torch.float32)
            for _ in range(LAUNCHES)]
    torch.cuda.synchronize()
    ref = outs[0].cpu().numpy()
    C, S = oracle_result(wl)
    assert_fp32(ref, C, S)
    for o in outs[1:]:
        assert np.array_equal(o.cpu().numpy().view(np.uint32), ref.view(np.uint32))
