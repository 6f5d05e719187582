"""The stall-injection build (liblowm_stress.so) must give the same bits.

The TensorRT-LLM PR "Fix two synchronization gaps in the MiniMax M3 low-M
split-K GEMM" (Hardware verification) found its ordering defects by stalling
chosen warps for 2 to 100 us, because a missing wait only shows when one
participant falls far behind.  The stress build stalls chosen wavefronts,
ranks and tiles with a bounded s_sleep loop at five sites:
  entry       before the first load (reorders which rank arrives last),
  stage read  after the stage barrier, before reading an LDS stage (a refill
              that did not wait for every reader would overwrite it),
  reduce      before a wavefront hands its sums to the wavefront reduction,
  publish     before a rank stores its partial and arrives,
  fold        in the owner, after its arrival, before reading the partials,
and one reordering site, late publish: the rank arrives first and stores its
partial only after the stall, as if its stores had landed that late (a rank
arrives without waiting for its stores' acknowledgement).
Every stalled launch must equal the unstalled launch of the default build
with the same tactic bit for bit (same kernels, same summation order), and so
stay within the oracle's bounds.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import split_bf16_gemm_amd as sbg
import workloads
from gpu_util import assert_bf16_launch, device, inputs, oracle_result, say, to_bits
from split_bf16_gemm_amd import binding

pytestmark = pytest.mark.gpu

DELAYS_NS = (2_000, 5_000, 10_000, 100_000)

# (sites, rank, wave, tile_mod, tile_sel, step)
PLANS = [
    ("entry rank 0", binding.SITE_ENTRY, 0, -1, 0, 0, -1),
    ("entry rank 1, every 3rd tile", binding.SITE_ENTRY, 1, -1, 3, 1, -1),
    ("stage read wave 1, every step", binding.SITE_STAGE_READ, -1, 1, 0, 0, -1),
    ("stage read wave 3, step 0", binding.SITE_STAGE_READ, -1, 3, 0, 0, 0),
    ("reduce wave 2", binding.SITE_REDUCE, -1, 2, 0, 0, -1),
    ("publish rank 0", binding.SITE_PUBLISH, 0, -1, 0, 0, -1),
    ("publish rank 1, odd tiles", binding.SITE_PUBLISH, 1, -1, 2, 1, -1),
    ("fold", binding.SITE_FOLD, -1, -1, 0, 0, -1),
    ("publish + fold, every 5th tile", binding.SITE_PUBLISH | binding.SITE_FOLD, -1, -1, 5, 2, -1),
]

# (workload, tactic): the default tactic at the headline shape is the line-pair
# tiles; the panel tiles run at M 64, split_k 2, the quarter tiles at M 16,
# split_k 2, the quarter-rows tiles at M 64, split_k 1 (each the default there).
CASES = [(workloads.HEADLINE, None), (workloads.HEADLINE, binding.tactic("lds", 16, 4, 2)),
         (workloads.HEADLINE, binding.tactic("reg", 16, 8, 2)),
         (workloads.by_name("sweep_m64_n6144_k4096_s2"), None),
         (workloads.by_name("sweep_m16_n6144_k4096_s2"), None),
         (workloads.by_name("sweep_m64_n6144_k4096_s1"), None)]


@pytest.fixture(scope="module")
def libs():
    device()
    stress = sbg.load("stress")
    yield sbg.load(), stress
    stress.configure_stress(0)


def launch(lib, ops, wl, tactic):
    A, W, ws = ops
    out = lib.gemm(A, W, wl.split_k, workspace=ws, tactic=tactic)
    torch.cuda.synchronize()
    return to_bits(out)


@pytest.mark.parametrize("case", CASES, ids=["line_default", "lds_ns2", "reg_u8_ns2", "panel_m64",
                                          "quarter_m16", "qrows_m64"])
@pytest.mark.parametrize("plan", PLANS, ids=[p[0] for p in PLANS])
def test_under_stalls(libs, plan, case):
    base, stress = libs
    wl, tactic = case
    dev = device()
    A, W = (t.to(dev) for t in inputs(wl))
    ws = base.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    ops = (A, W, ws)
    say("stress reference", plan[0], tactic)
    ref = launch(base, ops, wl, tactic)
    assert_bf16_launch(base, A, W, wl, ref, tactic=tactic, what="unstalled")
    name, sites, rank, wave, tmod, tsel, step = plan
    for d in DELAYS_NS:
        say("stress", name, d, "ns", tactic)
        stress.configure_stress(sites, rank, wave, tmod, tsel, step, d)
        try:
            got = launch(stress, ops, wl, tactic)
        finally:
            stress.configure_stress(0)
        assert np.array_equal(got, ref), f"{name}, {d} ns: output differs from the unstalled run"
    if ws is not None:
        assert not ws.cpu().numpy().any(), "the workspace (counters, partial slots) was left non-zero"


@pytest.mark.parametrize("wl", workloads.sweep(), ids=lambda w: w.name)
def test_sweep_in_stress_build(libs, wl):
    base, stress = libs
    dev = device()
    A, W = (t.to(dev) for t in inputs(wl))
    ws = base.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    ops = (A, W, ws)
    say("sweep reference", wl.name)
    ref = launch(base, ops, wl, None)
    assert_bf16_launch(base, A, W, wl, ref, what=wl.name)
    for sites, rank, wave, d in [(binding.SITE_PUBLISH, 0, -1, 10_000),
                                 (binding.SITE_ENTRY | binding.SITE_FOLD, -1, 0, 5_000),
                                 (binding.SITE_REDUCE, -1, 1, 2_000)]:
        say("sweep stress", wl.name, sites, rank, wave, d)
        stress.configure_stress(sites, rank, wave, 3, 0, -1, d)
        try:
            got = launch(stress, ops, wl, None)
        finally:
            stress.configure_stress(0)
        assert np.array_equal(got, ref), f"{wl.name}: stalls at {sites} changed the output"


def test_stress_library_without_stalls_matches(libs):
    base, stress = libs
    wl = workloads.SPLITK4
    dev = device()
    A, W = (t.to(dev) for t in inputs(wl))
    ws = base.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    say("stress lib, no stalls")
    assert np.array_equal(launch(base, (A, W, ws), wl, None), launch(stress, (A, W, ws), wl, None))


def _early_owners(stress, ops, wl):
    """Tiles whose last rank folded without arriving, from the stress build's
    per-workgroup timestamp trace of one launch (such a rank records an end
    but no arrival).  A traced launch measures timing only: its timestamp
    stores share the wait counter with the weight loads, so its output is
    not checked."""
    A, W, ws = ops
    tiles = (wl.N + 15) // 16
    grid = (tiles + 7) // 8 * 8 * wl.split_k
    T = stress.TRACE_SLOTS
    buf = torch.zeros(grid * T, dtype=torch.int64, device=A.device)
    stress.trace(buf)
    try:
        stress.gemm(A, W, wl.split_k, workspace=ws)
        torch.cuda.synchronize()
    finally:
        stress.trace(None)
    tr = buf.view(grid, T).cpu().numpy()
    return int(((tr[:, 5] > 0) & (tr[:, 4] == 0)).sum())


def test_last_rank_folds_early_and_its_poll_gives_up(libs):
    """At the headline shape the tile's last rank polls its peer's slot and,
    once the partial is there, folds without publishing or arriving.  With
    rank 0's publish stalled 100 us, past the poll's 20 us limit, no tile
    takes that path (the last rank publishes and arrives instead, and rank 0
    becomes the owner), and the output is unchanged bit for bit."""
    base, stress = libs
    wl = workloads.HEADLINE
    dev = device()
    A, W = (t.to(dev) for t in inputs(wl))
    ws = base.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    ops = (A, W, ws)
    say("early owner trace, no stall")
    ref = launch(base, ops, wl, None)
    assert _early_owners(stress, ops, wl) > 0, "no tile took the early-owner path"
    stress.configure_stress(binding.SITE_PUBLISH, 0, -1, 0, 0, -1, 100_000)
    try:
        say("early owner trace, rank 0 publish stalled 100 us")
        assert _early_owners(stress, ops, wl) == 0, "a last rank folded without its peer's partial"
        got = launch(stress, ops, wl, None)
    finally:
        stress.configure_stress(0)
    assert np.array_equal(got, ref), "the poll's time-out path changed the output"
    assert not ws.cpu().numpy().any(), "the workspace was left non-zero"


@pytest.mark.parametrize("rank", [0, 1, 2])
def test_split_k4_poll_gives_up_on_a_stalled_middle_rank(libs, rank):
    """split_k 4 (N 2304, K 12288): the last rank polls three peers.  One peer
    rank, on every other tile, stalls 100 us before publishing: the poll
    gives up after 20 us, the last rank publishes and arrives, and the
    stalled rank, arriving last, folds.  Tiles without the stall take the
    early path.  Every output bit must match the unstalled launch."""
    base, stress = libs
    wl = workloads.SPLITK4
    dev = device()
    A, W = (t.to(dev) for t in inputs(wl))
    ws = base.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    ops = (A, W, ws)
    say("split_k 4, stalled publish of rank", rank)
    ref = launch(base, ops, wl, None)
    stress.configure_stress(binding.SITE_PUBLISH, rank, -1, 2, 1, -1, 100_000)
    try:
        got = launch(stress, ops, wl, None)
    finally:
        stress.configure_stress(0)
    assert np.array_equal(got, ref), f"stalled rank {rank}: output differs"
    assert not ws.cpu().numpy().any(), "the workspace was left non-zero"


# (workload, tactic, late rank): every epilogue family (line-pair tiles with
# the early owner, the register ring's counter path, split_k 4, the strips of
# the panel and of the quarter tiles)
LATE_CASES = [(workloads.HEADLINE, None, 0), (workloads.HEADLINE, binding.tactic("reg", 16, 8, 2), 0),
              (workloads.SPLITK4, None, 1), (workloads.by_name("sweep_m64_n6144_k4096_s2"), None, 0),
              (workloads.by_name("sweep_m16_n6144_k4096_s2"), None, 1)]


@pytest.mark.parametrize("case", LATE_CASES, ids=["line_default", "reg_u8_ns2", "line_s4_rank1",
                                                  "panel_m64", "quarter_m16_rank1"])
def test_owner_rereads_a_partial_that_lands_after_the_arrival(libs, case):
    """One rank, on every other tile, arrives and stores its partial 200 us
    later.  The owner finds that slot still zero, re-reads it until the
    partial lands and folds it: the output equals the unstalled launch bit for
    bit, no tile is flagged, no counter is left open and the workspace is
    zero again."""
    base, stress = libs
    wl, tactic, rank = case
    dev = device()
    A, W = (t.to(dev) for t in inputs(wl))
    ws = base.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    ops = (A, W, ws)
    say("late publish reference", wl.name, tactic)
    ref = launch(base, ops, wl, tactic)
    stress.configure_stress(binding.SITE_LATE_PUBLISH, rank, -1, 2, 1, -1, 200_000)
    try:
        say("late publish 200 us, rank", rank, wl.name, tactic)
        got = launch(stress, ops, wl, tactic)
    finally:
        stress.configure_stress(0)
    assert np.array_equal(got, ref), "a partial that landed late changed the output"
    assert base.workspace_status(ws, wl.N) == (0, 0), "a tile was flagged or left open"
    assert not ws.cpu().numpy().any(), "the workspace was left non-zero"


def test_owner_gives_up_past_its_bound_and_flags_the_tile(libs):
    """Rank 0 of every 4th tile at the headline shape arrives and stores its
    partial 3 ms later, past the owner's 1 ms bound.  Every owner that gives
    up sets its tile's fault word, which lowm_workspace_status reports; no
    counter is left open and the other tiles' outputs are unchanged.  Zeroing
    the workspace clears the flags and the next launch is exact again."""
    base, stress = libs
    wl = workloads.HEADLINE
    dev = device()
    A, W = (t.to(dev) for t in inputs(wl))
    ws = base.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    ops = (A, W, ws)
    say("give-up reference")
    ref = launch(base, ops, wl, None)
    tiles = (wl.N + 15) // 16
    selected = np.arange(tiles) % 4 == 1
    stress.configure_stress(binding.SITE_LATE_PUBLISH, 0, -1, 4, 1, -1, 3_000_000)
    try:
        say("late publish 3 ms, rank 0, every 4th tile")
        got = launch(stress, ops, wl, None)
    finally:
        stress.configure_stress(0)
    faulted, open_ = base.workspace_status(ws, wl.N)
    assert open_ == 0, "a counter was left open"
    assert 1 <= faulted <= int(selected.sum()), f"{faulted} tiles flagged"
    keep = np.repeat(~selected, 16)[:wl.N]
    assert np.array_equal(got[:, keep], ref[:, keep]), "an unstalled tile's output changed"
    ws.zero_()
    assert base.workspace_status(ws, wl.N) == (0, 0)
    say("after zeroing the workspace")
    assert np.array_equal(launch(base, ops, wl, None), ref), "the launch after recovery differs"
