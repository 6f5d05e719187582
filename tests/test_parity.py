"""Parity of the HIP path with the fp64 oracle, element by element.

Bars (tests/checks.py): integer-valued inputs bit-exact in fp32 and bf16;
random inputs fp32 within 1e-3 * sum|a||w| and bf16 within one ulp of the
oracle's round-to-nearest-even value.  Shapes: the integer closed form of the
Triton issue "warpgroup_mma_wait does not properly synchronize across
warpgroups" (Describe the bug), the three shapes of the TensorRT-LLM PR "Fix
two synchronization gaps in the MiniMax M3 low-M split-K GEMM" (Hardware
verification) at full size in the launch configuration the benchmark times,
the M x split_k sweep, ragged tails and every tactic the build provides.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import split_bf16_gemm_amd as sbg
import workloads
from checks import assert_bf16, assert_exact_integer, assert_fp32
from gpu_util import (all_tactics, device, quarter_built, inputs, oracle_result, report, run,
                      say, to_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    device()
    return sbg.load()


def check_random(lib, wl, tactic=None, what=""):
    A, W = inputs(wl)
    C, S = oracle_result(wl)
    say(what or wl.name, wl.M, wl.N, wl.K, wl.split_k, tactic)
    c32 = run(lib, A, W, wl.split_k, f32out=True, tactic=tactic)
    if c32 is None:
        return None
    c16 = run(lib, A, W, wl.split_k, f32out=False, tactic=tactic)
    c32 = c32.numpy()
    b16 = to_bits(c16)
    assert_fp32(c32, C, S, what=what or wl.name)
    v = assert_bf16(b16, C, S, wl.K, oracle.default(), c32, what=what or wl.name)
    # the two entry points share the kernel and its order: bf16 = RNE(fp32)
    assert np.array_equal(b16, oracle.round_bf16(c32.astype(np.float64))), what
    report(what or wl.name, v, C.size)
    return v


def test_closed_form_bit_exact_every_tactic(lib):
    wl = workloads.INT_EXACT
    A, W = inputs(wl)
    C, _ = oracle_result(wl)
    ran = 0
    for t in all_tactics(wl.M):
        say("closed form", t)
        c32 = run(lib, A, W, wl.split_k, f32out=True, tactic=t)
        if c32 is None:
            continue
        c16 = run(lib, A, W, wl.split_k, f32out=False, tactic=t)
        assert_exact_integer(c32.numpy(), to_bits(c16), C, oracle.default(), what=repr(t))
        ran += 1
    assert ran >= 8


def test_closed_form_default_tactic(lib):
    wl = workloads.INT_EXACT
    A, W = inputs(wl)
    C, _ = oracle_result(wl)
    say("closed form default")
    c32 = run(lib, A, W, wl.split_k, f32out=True)
    c16 = run(lib, A, W, wl.split_k)
    assert_exact_integer(c32.numpy(), to_bits(c16), C, oracle.default(), what="default")


@pytest.mark.parametrize("M,N,K", [(5, 100, 384), (16, 64, 1024), (33, 48, 512), (64, 40, 256)])
def test_integer_inputs_identical_for_every_split(lib, M, N, K):
    wl = workloads.Workload("int_both", M, N, K, 1, kind="int_both", seed_a=M, seed_w=N)
    A, W = inputs(wl)
    C, _ = oracle_result(wl)
    first = None
    for s in (1, 2, 4, 8):
        say("integer split", M, N, K, s)
        c32 = run(lib, A, W, s, f32out=True)
        c16 = run(lib, A, W, s)
        assert_exact_integer(c32.numpy(), to_bits(c16), C, oracle.default(), what=f"S={s}")
        if first is None:
            first = to_bits(c16)
        assert np.array_equal(first, to_bits(c16))


@pytest.mark.parametrize("wl", [workloads.HEADLINE, workloads.SPLITK4, workloads.WIDE_N],
                         ids=lambda w: w.name)
def test_full_size_pages_shapes(lib, wl):
    check_random(lib, wl)


@pytest.mark.parametrize("wl", workloads.sweep(), ids=lambda w: w.name)
def test_sweep(lib, wl):
    check_random(lib, wl)


RAGGED = [
    (1, 1, 8, 1), (1, 1, 16, 2), (3, 17, 64, 2), (4, 15, 32, 4), (5, 1000, 1032, 1),
    (7, 257, 1032, 3), (17, 33, 520, 5), (31, 16, 64, 8), (48, 127, 4104, 3),
    (63, 77, 2048, 8), (64, 65, 96, 4), (2, 4097, 40, 5), (9, 300, 8, 1),
]


@pytest.mark.parametrize("M,N,K,S", RAGGED)
def test_ragged(lib, M, N, K, S):
    wl = workloads.Workload(f"ragged_{M}_{N}_{K}_{S}", M, N, K, S,
                            seed_a=M * 7 + S, seed_w=N * 3 + K)
    check_random(lib, wl)


# The largest split_k the boundary accepts (one 16-byte vector of K per rank
# at K 2048: 256 ranks per tile on the generic fold) and a long K at split_k
# 64, from one activation row to the largest M.
LARGEST_SPLIT = [
    (1, 64, 2048, sbg.binding.MAX_SPLIT_K), (4, 300, 2048, sbg.binding.MAX_SPLIT_K),
    (64, 100, 4096, sbg.binding.MAX_SPLIT_K), (16, 1000, 16384, 64),
]


@pytest.mark.parametrize("M,N,K,S", LARGEST_SPLIT)
def test_largest_split_k(lib, M, N, K, S):
    wl = workloads.Workload(f"split{S}_{M}_{N}_{K}", M, N, K, S,
                            seed_a=M + 1100, seed_w=N + K)
    check_random(lib, wl)


def _drawn_shapes(n=16, seed=2024):
    """Shapes drawn from a fixed seed over the whole supported range: M 1..64,
    N 1..3000 (mostly ragged), split_k 1..16, K a multiple of 8 * split_k up
    to 4096 (slices that are whole line pairs, whole 64-K steps, or neither)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 65))
        N = int(rng.integers(1, 3001))
        S = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 16]))
        K = 8 * S * int(rng.integers(1, 4096 // (8 * S) + 1))
        out.append((M, N, K, S))
    return out


@pytest.mark.parametrize("M,N,K,S", _drawn_shapes())
def test_drawn_shapes_default_tactic(lib, M, N, K, S):
    wl = workloads.Workload(f"drawn_{M}_{N}_{K}_{S}", M, N, K, S, seed_a=M + N, seed_w=K + S)
    check_random(lib, wl)


QROWS_CASES = [  # M, N, K: ragged M (a short last block), ragged N, every tile width
    (64, 2048, 4096), (48, 3072, 4096), (33, 1000, 2048), (63, 777, 1024),
    (40, 100, 512), (64, 520, 4096),
]


@pytest.mark.parametrize("M,N,K", QROWS_CASES)
def test_quarter_rows_tiles(lib, M, N, K):
    """Quarter-rows tiles (split_k 1): blocks of 16..64 activation rows per
    workgroup and tiles of 16..64 columns.  Each is judged against the oracle
    and must give the bits of the quarter tiles, whose kernel and summation
    order it shares, in both output types."""
    wl = workloads.Workload(f"qrows_{M}_{N}_{K}", M, N, K, 1, seed_a=M + 500, seed_w=N + 600)
    A, W = inputs(wl)
    ref = {}
    for f32 in (False, True):
        for rows, ring in ((32, 3), (16, 3), (64, 2)):
            ref[f32] = run(lib, A, W, 1, f32out=f32, tactic=sbg.tactic("quarter", rows, 2, ring))
            if ref[f32] is not None:
                break
        assert ref[f32] is not None
    ran = 0
    for blocks in (1, 2, 3, 4):
        for rows, ring in ((16, 4), (32, 3), (48, 3), (64, 3)):
            t = sbg.tactic("qrows", rows, blocks, ring)
            if check_random(lib, wl, tactic=t, what=f"{wl.name} {t!r}") is None:
                continue
            for f32 in (False, True):
                got = run(lib, A, W, 1, f32out=f32, tactic=t)
                assert torch.equal(got.view(torch.int32) if f32 else got.view(torch.int16),
                                   ref[f32].view(torch.int32) if f32 else ref[f32].view(torch.int16)), \
                    f"{t!r} differs from the quarter tiles (f32={f32})"
            ran += 1
    assert ran >= 8, ran


@pytest.mark.parametrize("M,N,K", [(49, 6144, 4096), (57, 3000, 2048), (63, 100, 1024),
                                   (50, 4096, 8192)])
def test_quarter_rows_by_default(lib, M, N, K):
    """49..63 rows without split-K: the default tactic is the quarter-rows
    tiles with a short second row block; judged against the oracle."""
    t = lib.pick_tactic(M, N, K, 1)
    assert t.stage == sbg.binding.LOWM_STAGE_QUARTER_ROWS, t
    wl = workloads.Workload(f"qrows_default_{M}_{N}_{K}", M, N, K, 1, seed_a=M + 700, seed_w=N + 800)
    check_random(lib, wl)


def test_every_tactic_random(lib):
    """M 20 (two row blocks) with whole 256-K slices: every tactic family
    applies (5 register/LDS variants at 16 rows, 4 at 32, 3 line-pair rings,
    3 panel rings at 64 rows and 3 at 32, 3 quarter rings at 16 and 32 rows
    and 2 at 64)."""
    wl = workloads.Workload("tactics", 20, 300, 2048, 2, seed_a=77, seed_w=78)
    ran = []
    for t in all_tactics(wl.M):
        if check_random(lib, wl, tactic=t, what=repr(t)) is not None:
            ran.append(t)
    assert len(ran) == 26, ran


def test_every_tactic_small_m_ragged_k(lib):
    """K / split_k = 344 is neither whole line pairs per wavefront nor whole
    64-K steps, and M 4 is one row block: the register rings of 4 and 8
    chunks and both LDS rings run at 16 and 32 rows (8 tactics); the
    line-pair, panel and quarter tiles (whole 64-K steps per wavefront), and
    the 16-chunk register ring (too many registers), return
    LOWM_ERR_UNSUPPORTED."""
    wl = workloads.Workload("tactics_k", 4, 97, 1032, 3, seed_a=5, seed_w=6)
    ran = []
    for t in all_tactics(wl.M):
        if check_random(lib, wl, tactic=t, what=repr(t)) is not None:
            ran.append(t)
    stages = sorted({t.stage for t in ran})
    assert stages == [sbg.binding.LOWM_STAGE_LDS, sbg.binding.LOWM_STAGE_REG], ran
    assert len(ran) == 8, ran


def test_workspace_returns_to_zero_and_guard_intact(lib):
    dev = device()
    wl = workloads.HEADLINE
    A, W = inputs(wl)
    need = lib.workspace_bytes(wl.M, wl.N, wl.K, wl.split_k)
    guard = 4096
    ws = torch.zeros(need + guard, dtype=torch.uint8, device=dev)
    ws[need:] = 0xA5
    say("counters/guard")
    for _ in range(3):
        run(lib, A, W, wl.split_k, workspace=ws)
    host = ws.cpu().numpy()
    ctr = host[:sbg.counter_bytes(wl.N)]
    assert not ctr.any(), "an arrival counter was left non-zero"
    assert not host[:need].any(), "a partial slot was left non-zero"
    assert (host[need:] == 0xA5).all(), "the kernel wrote past the workspace"


def test_workspace_status_reads_the_counter_lines(lib):
    """lowm_workspace_status counts the tiles whose fault word (word 1 of
    their 256-byte counter line) or arrival count (word 0) is non-zero; the
    words are planted from the host, then a launch on a clean workspace
    leaves both counts at zero."""
    dev = device()
    wl = workloads.HEADLINE
    ws = lib.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    words = ws.view(torch.int32)
    words[64 * 3 + 1] = 1          # tile 3: fault word
    words[64 * 5] = 1              # tile 5: open arrival count
    words[64 * 7 + 1] = 1          # tile 7: both
    words[64 * 7] = 2
    assert lib.workspace_status(ws, wl.N) == (2, 2)
    ws.zero_()
    A, W = inputs(wl)
    say("status after a launch")
    run(lib, A, W, wl.split_k, workspace=ws)
    assert lib.workspace_status(ws, wl.N) == (0, 0)


def test_split_one_needs_no_workspace(lib):
    wl = workloads.Workload("s1", 4, 640, 1024, 1, seed_a=1, seed_w=2)
    A, W = inputs(wl)
    C, S = oracle_result(wl)
    say("split 1, no workspace")
    out = lib.gemm(A.to(device()), W.to(device()), 1, workspace=None,
                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_fp32(out.cpu().numpy(), C, S)


def test_launch_is_asynchronous_on_the_given_stream(lib):
    dev = device()
    wl = workloads.HEADLINE
    A, W = (t.to(dev) for t in inputs(wl))
    ws = lib.make_workspace(wl.M, wl.N, wl.K, wl.split_k, dev)
    s = torch.cuda.Stream(device=dev)
    say("side stream")
    with torch.cuda.stream(s):
        out = lib.gemm(A, W, wl.split_k, workspace=ws, out_dtype=torch.float32)
    s.synchronize()
    C, S = oracle_result(wl)
    assert_fp32(out.cpu().numpy(), C, S)


def test_one_workspace_serves_launches_of_different_shapes(lib):
    """Every launch returns the whole workspace to zero, so one buffer, sized
    for the largest shape, serves launches of any shape in turn, early-owner
    shapes (the last rank reads its peers' slots without the counter) after
    counter-only ones and back, each bit-identical to a launch on a fresh
    workspace."""
    dev = device()
    shapes = [workloads.Workload("ws_a", 4, 6144, 4096, 2, seed_a=31, seed_w=32),
              workloads.Workload("ws_b", 16, 2304, 4096, 8, seed_a=33, seed_w=34),
              workloads.Workload("ws_c", 2, 1000, 3072, 3, seed_a=35, seed_w=36),
              workloads.Workload("ws_d", 64, 768, 2048, 4, seed_a=37, seed_w=38)]
    need = max(lib.workspace_bytes(w.M, w.N, w.K, w.split_k) for w in shapes)
    shared = torch.zeros(need, dtype=torch.uint8, device=dev)
    fresh = {}
    for wl in shapes:
        A, W = inputs(wl)
        fresh[wl.name] = to_bits(run(lib, A, W, wl.split_k))
    say("shared workspace, mixed shapes")
    for wl in shapes + shapes[::-1]:
        A, W = inputs(wl)
        got = to_bits(run(lib, A, W, wl.split_k, workspace=shared))
        assert np.array_equal(got, fresh[wl.name]), f"{wl.name} differs on the shared workspace"
        assert not shared.cpu().numpy().any(), f"{wl.name} left the shared workspace non-zero"


PANEL_CASES = [  # M, N, K, S: ragged N (partial strips, wavefronts past the end),
    (17, 130, 640, 5),     # 2 steps per slice (ring not filled), generic split_k fold
    (33, 77, 512, 2),      # 2 tiles: the second has one partial strip
    (48, 1000, 1536, 3),   # 3 activation blocks
    (64, 64, 4096, 8),     # one tile, split_k 8
    (64, 6200, 2048, 1),   # no split: direct stores
    (32, 2304, 12288, 4),  # long slices
]


@pytest.mark.parametrize("rows,ring", [(64, 3), (64, 4), (64, 6), (32, 3), (32, 4), (32, 6)])
@pytest.mark.parametrize("M,N,K,S", PANEL_CASES)
def test_panel_tiles(lib, M, N, K, S, rows, ring):
    """Panel tiles (activation panel shared in LDS, each 16-column strip
    owned by one wavefront, or with 32-row tiles by two that split the K
    slice in halves, through the exchange) against the oracle.  With 32-row
    tiles the ring of 6 does not fit LDS for 49..64 rows."""
    wl = workloads.Workload(f"panel_{M}_{N}_{K}_{S}", M, N, K, S, seed_a=M + ring, seed_w=N + S)
    t = sbg.tactic("panel", rows, 2, ring)
    if rows == 32 and ring == 6 and M > 48:
        assert lib.check_launch(M, N, K, S, tactic=t) == sbg.binding.LOWM_ERR_UNSUPPORTED
        return
    v = check_random(lib, wl, tactic=t, what=f"panel {rows}:{ring} {M}x{N}x{K} s{S}")
    assert v is not None, f"panel {rows} ring {ring} is not built for M {M}"


@pytest.mark.parametrize("wl", [w for w in workloads.sweep() if w.M >= 32], ids=lambda w: w.name)
def test_panel_tiles_sweep(lib, wl):
    v = check_random(lib, wl, tactic=sbg.tactic("panel", 64, 2, 4), what=f"panel {wl.name}")
    assert v is not None


QUARTER_CASES = [  # M, N, K, S
    (17, 130, 1280, 5),    # K slice 256: one step per wavefront, generic split_k fold
    (33, 77, 512, 2),      # ragged N: partial strips, wavefronts past the end
    (48, 1000, 1536, 3),   # 3 activation blocks, 2 steps per wavefront
    (64, 64, 4096, 8),     # one tile, split_k 8
    (64, 6200, 2048, 1),   # no split: direct stores, 8 steps per wavefront
    (32, 2304, 12288, 4),  # long slices: 12 steps per wavefront
    (5, 1000, 2048, 2),    # one activation block
]


@pytest.mark.parametrize("rows,ring", [(r, d) for r in (16, 32, 64) for d in (2, 3, 4)])
@pytest.mark.parametrize("M,N,K,S", QUARTER_CASES)
def test_quarter_tiles(lib, M, N, K, S, rows, ring):
    """Quarter tiles (each wavefront one quarter of the K slice for every row
    of the tile, both operands through its own LDS ring, quarter sums added
    in order through LDS, then the strip epilogue) against the oracle, where
    the build provides them; elsewhere the launch is LOWM_ERR_UNSUPPORTED."""
    wl = workloads.Workload(f"quarter_{M}_{N}_{K}_{S}", M, N, K, S, seed_a=M + ring, seed_w=N + S)
    t = sbg.tactic("quarter", rows, 2, ring)
    if not quarter_built(M, rows, ring):
        assert lib.check_launch(M, N, K, S, tactic=t) == sbg.binding.LOWM_ERR_UNSUPPORTED
        return
    v = check_random(lib, wl, tactic=t, what=f"quarter {rows}:{ring} {M}x{N}x{K} s{S}")
    assert v is not None, f"quarter {rows} ring {ring} is not built for M {M}"
