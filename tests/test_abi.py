"""The C ABI of include/lowm.h, host side only (no kernel is launched).

Every function the header declares is exported by the built libraries, and
argument validation returns its documented error before any HIP call: these
tests hand in fake non-NULL pointers that must never reach a launch.
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import pytest

import split_bf16_gemm_amd as sbg
from split_bf16_gemm_amd import binding

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "lowm.h"

FAKE = 0x10000      # 16-byte aligned, never dereferenced
FAKE_ODD = 0x10002  # 2-byte aligned only
# Disjoint fake buffers for calls that must get past the host's overlap check
# (16 MiB apart: far beyond any span these tests describe).
FAKE_A, FAKE_W, FAKE_C, FAKE_WS = 0x1000000, 0x2000000, 0x3000000, 0x4000000


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(lowm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sbg.load()


@pytest.fixture(scope="module")
def stress_lib():
    return sbg.load("stress")


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("lowm_gemm_splitk", "lowm_gemm_splitk_f32out",
              "lowm_gemm_splitk_workspace_bytes", "lowm_strerror", "lowm_last_hip_error"):
        assert n in names


@pytest.mark.parametrize("kind", ["default", "stress"])
def test_every_declared_symbol_is_exported(kind):
    lib = sbg.load(kind)
    for name in declared_functions():
        assert hasattr(lib.lib, name), f"{lib.path.name} does not export {name}"


def test_stress_build_has_its_hook(lib, stress_lib):
    assert stress_lib.has_stress
    assert not lib.has_stress


def test_strerror_names_every_code(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.strerror(code) and "unknown" not in lib.strerror(code)
    assert "unknown" in lib.strerror(-99)


def test_workspace_bytes(lib):
    assert lib.workspace_bytes(4, 6144, 4096, 1) == 0
    # a 256-byte line per counter, ceil(N/16) counters, then S*M*round_up(N, 64) fp32
    assert lib.workspace_bytes(4, 6144, 4096, 2) == 384 * 256 + 2 * 4 * 6144 * 4
    assert lib.workspace_bytes(4, 2304, 12288, 4) == 144 * 256 + 4 * 4 * 2304 * 4
    assert lib.workspace_bytes(3, 17, 64, 2) == 2 * 256 + 2 * 3 * 64 * 4
    assert lib.workspace_bytes(4, 512, 1024, 3) == 0          # K % (8*3) != 0
    assert lib.workspace_bytes(65, 512, 1024, 2) == 0         # M > 64
    assert lib.workspace_bytes(0, 512, 1024, 2) == 0
    assert sbg.counter_bytes(6144) == 384 * 256
    assert sbg.counter_bytes(17) == 2 * 256


def test_binding_counter_region_matches_the_library(lib):
    # the partials start right after the counters: workspace = counters + partials
    for N in (1, 15, 16, 17, 64, 100, 2304, 6144, 49152):
        for (M, S) in ((1, 2), (4, 2), (16, 8), (64, 3)):
            K = 8 * S * 4
            parts = S * M * ((N + 63) // 64 * 64) * 4
            assert lib.workspace_bytes(M, N, K, S) == sbg.counter_bytes(N) + parts, (M, N, S)
            assert sbg.counter_bytes(N) % 256 == 0


def test_pick_tactic_is_valid_for_every_workload(lib):
    import workloads
    for wl in workloads.ALL:
        t = lib.pick_tactic(wl.M, wl.N, wl.K, wl.split_k)
        assert t.rows in (16, 32, 48, 64) and t.waves == 4
        if t.stage in (binding.LOWM_STAGE_REG, binding.LOWM_STAGE_LDS):
            assert t.rows >= min(32, 16 * ((wl.M + 15) // 16))
        assert lib.check_launch(wl.M, wl.N, wl.K, wl.split_k, tactic=t) == 0


def test_pick_line_pairs_for_four_rows_or_fewer_with_split(lib):
    line = binding.LOWM_STAGE_LINE
    t = lib.pick_tactic(4, 6144, 4096, 2)        # 8 line pairs per wavefront
    assert (t.stage, t.rows, t.unroll, t.stages) == (line, 16, 2, 4)
    t = lib.pick_tactic(1, 6144, 4096, 8)        # 2 pairs
    assert (t.stage, t.rows, t.stages) == (line, 16, 2)
    t = lib.pick_tactic(4, 2304, 12288, 4)       # 12 pairs
    assert (t.stage, t.rows, t.stages) == (line, 16, 4)
    t = lib.pick_tactic(4, 97, 1032, 3)          # ragged K slice: register ring
    assert t.stage == binding.LOWM_STAGE_REG


def test_pick_panel_tiles_above_32_rows_with_split_or_split_k_4(lib):
    panel = binding.LOWM_STAGE_PANEL
    # 64-row tiles; without split-K only where the K slice is not whole 64-K
    # steps per wavefront (no quarter tiles)
    for M, N, K, S, rows in [(64, 6144, 4096, 2, 64), (64, 49152, 4096, 8, 64),
                             (40, 6144, 4096, 4, 64),
                             (33, 2304, 12288, 4, 64), (64, 6144, 1088, 1, 64),
                             (17, 6144, 4096, 4, 64), (32, 1536, 8192, 8, 64)]:
        t = lib.pick_tactic(M, N, K, S)
        assert (t.stage, t.rows, t.unroll, t.stages) == (panel, rows, 2, 4), (M, N, K, S, t)
    # a slice that is not whole 64-K steps: register ring
    t = lib.pick_tactic(64, 6144, 1032, 3)
    assert t.stage == binding.LOWM_STAGE_REG
    # 16 rows or fewer: never panel tiles (the build has none for one row block)
    for M in (1, 4, 16):
        assert lib.pick_tactic(M, 6144, 4096, 2).stage != panel
        assert lib.check_launch(M, 6144, 4096, 2, tactic=binding.tactic("panel", 64, 2, 4)) == \
            binding.LOWM_ERR_UNSUPPORTED


def test_pick_quarter_tiles_where_measured_faster(lib):
    """Quarter tiles: split_k 1 for every M; 5..16 rows with any split_k;
    17..32 rows with split_k 2.  The tile width and ring follow the number
    of workgroups and rows."""
    quarter = binding.LOWM_STAGE_QUARTER
    for M, N, K, S, rows, ring in [
            (16, 6144, 4096, 1, 32, 4), (8, 6144, 4096, 1, 32, 4), (1, 6144, 4096, 1, 32, 4),
            (4, 8192, 4096, 1, 32, 4),       # 256 32-row workgroups: ring 4
            (4, 24576, 4096, 1, 32, 3),      # 768: ring 3 fits two per CU
            (8, 6144, 4096, 2, 48, 3),       # 384 32-row, 256 48-row workgroups
            (8, 12288, 4096, 2, 48, 2),      # 512 48-row workgroups: two rounds
            (16, 6144, 4096, 4, 48, 2),      # 768 32-row, 512 48-row workgroups
            (16, 1536, 8192, 2, 16, 3),      # 96
            (8, 1536, 8192, 4, 32, 3),       # 192
            (12, 6144, 4096, 8, 32, 2),      # split_k 8: 32-row tiles, ring 2
            (32, 6144, 4096, 1, 32, 4),      # 384 16-row workgroups
            (24, 6144, 4096, 2, 48, 3),      # 256 48-row workgroups
            (24, 12288, 4096, 2, 48, 3),     # fewest rounds x rows: 48 rows, two rounds
            (24, 24576, 4096, 2, 64, 3),     # 64 rows, three rounds
            (32, 3072, 4096, 2, 32, 3),      # one round of 32-row workgroups
            (32, 1536, 8192, 2, 16, 3),      # 192 16-row workgroups
            (20, 3072, 4096, 1, 16, 3),
            (64, 8192, 4096, 1, 32, 3),      # 256 32-row workgroups
            (64, 12288, 4096, 1, 48, 2),     # 256 48-row workgroups: one round
            (64, 16384, 4096, 1, 64, 2),     # 256 64-row workgroups
            (64, 24576, 4096, 1, 48, 2),     # two rounds of 48-row tiles
            (40, 6144, 4096, 1, 32, 3),      # 33..48 rows: no quarter-rows tiles
            (48, 3072, 4096, 1, 16, 3),      # 192 16-row workgroups
            (48, 24576, 4096, 1, 48, 3),     # two rounds of 48-row tiles
            (40, 12288, 4096, 1, 48, 3),
            (32, 24576, 4096, 1, 32, 4),     # up to 32 rows: 32-row tiles
            (48, 100, 512, 1, 16, 3)]:
        t = lib.pick_tactic(M, N, K, S)
        assert (t.stage, t.rows, t.unroll, t.stages) == (quarter, rows, 2, ring), (M, N, K, S, t)
    # not whole 64-K steps per wavefront, four rows or fewer with split-K,
    # more than 32 rows with split-K, or 17..32 rows with split_k 4: other
    # tiles
    for M, N, K, S in [(16, 6144, 4160, 1), (4, 6144, 4096, 2), (64, 6144, 4096, 2),
                       (32, 6144, 4096, 4)]:
        assert lib.pick_tactic(M, N, K, S).stage != quarter, (M, N, K, S)


def test_pick_quarter_rows_for_33_to_64_rows_without_split(lib):
    """49..64 rows, split_k 1: two workgroups per tile (one per 32-row block)
    and the narrowest tile width (up to 48 columns) whose blocks fit the 256
    CUs once; wider shapes and 33..48 rows keep the quarter tiles.  Never
    with split-K or for the push epilogue's tile choice."""
    qrows = binding.LOWM_STAGE_QUARTER_ROWS
    for M, N, K, rows, ring in [
            (64, 2048, 4096, 16, 4),        # 128 tiles x 2 blocks
            (64, 4096, 4096, 32, 3),        # 128 x 2
            (64, 6144, 4096, 48, 3),        # 128 x 2
            (49, 6144, 4096, 48, 3),        # a second block of 17 rows
            (56, 3072, 4096, 32, 3),        # 96 x 2
            (64, 2304, 12288, 32, 3),       # 72 x 2
            (64, 100, 512, 16, 4)]:
        t = lib.pick_tactic(M, N, K, 1)
        assert (t.stage, t.rows, t.unroll, t.stages) == (qrows, rows, 2, ring), (M, N, K, t)
        assert lib.check_launch(M, N, K, 1, tactic=t) == binding.LOWM_OK
        assert lib.check_launch(M, N, K, 1, f32out=True, tactic=t) == binding.LOWM_OK
    for M, N, K, S in [(64, 12288, 4096, 1), (64, 8192, 4096, 1), (64, 6144, 4096, 2),
                       (48, 2048, 4096, 1), (32, 6144, 4096, 1), (16, 2048, 4096, 1),
                       (64, 6144, 1088, 1)]:
        assert lib.pick_tactic(M, N, K, S).stage != qrows, (M, N, K, S)
    # the family exists only without split-K
    t = binding.tactic("qrows", 48, 2, 3)
    assert lib.check_launch(64, 6144, 4096, 2, tactic=t) == binding.LOWM_ERR_UNSUPPORTED
    # blocks of 16..64 rows, none wider than the build's quarter tiles
    assert lib.check_launch(64, 6144, 4096, 1, tactic=binding.tactic("qrows", 48, 1, 3)) == 0
    assert lib.check_launch(64, 6144, 4096, 1, tactic=binding.tactic("qrows", 48, 5, 3)) == \
        binding.LOWM_ERR_UNSUPPORTED


def call(lib, A=FAKE_A, W=FAKE_W, C=FAKE_C, M=4, N=64, K=256, S=2, ws=FAKE_WS, f32=False,
         tac=None):
    return lib.call_raw(A, W, C, M, N, K, S, ws, 0, f32out=f32, tactic=tac)


@pytest.mark.parametrize("f32", [False, True])
def test_invalid_arguments(lib, f32):
    assert call(lib, A=0, f32=f32) == binding.LOWM_ERR_INVALID_ARG
    assert call(lib, W=0, f32=f32) == binding.LOWM_ERR_INVALID_ARG
    assert call(lib, C=0, f32=f32) == binding.LOWM_ERR_INVALID_ARG
    assert call(lib, M=0, f32=f32) == binding.LOWM_ERR_INVALID_ARG
    assert call(lib, N=-1, f32=f32) == binding.LOWM_ERR_INVALID_ARG
    assert call(lib, K=0, f32=f32) == binding.LOWM_ERR_INVALID_ARG
    assert call(lib, S=0, f32=f32) == binding.LOWM_ERR_INVALID_ARG


@pytest.mark.parametrize("f32", [False, True])
def test_unsupported(lib, f32):
    assert call(lib, M=65, f32=f32) == binding.LOWM_ERR_UNSUPPORTED
    assert call(lib, K=260, f32=f32) == binding.LOWM_ERR_UNSUPPORTED       # K % 16 != 0
    assert call(lib, S=257, K=8 * 257, f32=f32) == binding.LOWM_ERR_UNSUPPORTED
    assert call(lib, A=FAKE_A + 8, f32=f32) == binding.LOWM_ERR_UNSUPPORTED
    assert call(lib, W=FAKE_W + 4, f32=f32) == binding.LOWM_ERR_UNSUPPORTED
    assert call(lib, ws=FAKE_WS + 8, f32=f32) == binding.LOWM_ERR_UNSUPPORTED
    assert call(lib, C=FAKE_C + 1, f32=f32) == binding.LOWM_ERR_UNSUPPORTED


def test_fp32_output_needs_4_byte_alignment(lib):
    assert call(lib, C=FAKE_C + 2, f32=True) == binding.LOWM_ERR_UNSUPPORTED


@pytest.mark.parametrize("f32", [False, True])
def test_overlapping_buffers_are_rejected(lib, f32):
    """An output whose bytes meet an operand, another output or the
    workspace (or a workspace that meets an operand) is an invalid argument,
    found on the host before any HIP call.  M 4, N 64, K 256: A spans 2 KiB,
    W 32 KiB, C 512 B (bf16) or 1 KiB (fp32)."""
    E = binding
    c_bytes = 4 * 64 * (4 if f32 else 2)
    assert call(lib, C=FAKE_A, f32=f32) == E.LOWM_ERR_INVALID_ARG
    assert call(lib, C=FAKE_A + 2048 - 4, f32=f32) == E.LOWM_ERR_INVALID_ARG     # A's last bytes
    assert call(lib, C=FAKE_W - c_bytes + 4, f32=f32) == E.LOWM_ERR_INVALID_ARG  # W's first bytes
    assert call(lib, C=FAKE_W + 32768 - 4, f32=f32) == E.LOWM_ERR_INVALID_ARG    # W's last bytes
    assert call(lib, C=FAKE_WS, f32=f32) == E.LOWM_ERR_INVALID_ARG
    assert call(lib, ws=FAKE_A, f32=f32) == E.LOWM_ERR_INVALID_ARG
    assert call(lib, ws=FAKE_W + 16, f32=f32) == E.LOWM_ERR_INVALID_ARG
    assert call(lib, ws=FAKE_C - 16, f32=f32) == E.LOWM_ERR_INVALID_ARG          # runs into C
    assert lib.lib.lowm_last_hip_error() == 0


def test_workspace_required_for_split(lib):
    assert call(lib, ws=0) == binding.LOWM_ERR_WORKSPACE
    assert call(lib, ws=0, f32=True) == binding.LOWM_ERR_WORKSPACE


def test_unknown_tactic_is_unsupported(lib):
    bad = [binding.tactic("reg", 80, 4, 3), binding.tactic("reg", 16, 3, 3),
           binding.tactic("lds", 16, 2, 5), binding.tactic("reg", 16, 4, 3, waves=8)]
    for t in bad:
        assert call(lib, tac=t) == binding.LOWM_ERR_UNSUPPORTED, t


def test_errors_precede_any_hip_call(lib):
    # validation failures leave no HIP error behind
    call(lib, M=0)
    assert lib.lib.lowm_last_hip_error() == 0


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        binding.Library(tmp_path / "liblowm.so")


def test_pick_tactic_rejects_bad_sizes(lib):
    t = binding.Tactic()
    assert lib.lib.lowm_pick_tactic(65, 64, 256, 1, ctypes.byref(t)) == binding.LOWM_ERR_UNSUPPORTED
    assert lib.lib.lowm_pick_tactic(4, 64, 256, 0, ctypes.byref(t)) == binding.LOWM_ERR_INVALID_ARG
    assert lib.lib.lowm_pick_tactic(4, 64, 256, 1, None) == binding.LOWM_ERR_INVALID_ARG


def test_default_tactic_is_launchable_for_every_shape(lib):
    # every M 1..64 with several K/split_k mixes: the default tactic must have
    # an instantiation in both output types (the launch must not refuse it)
    failures = []
    for M in range(1, 65):
        for (K, S) in [(512, 1), (512, 2), (1024, 8), (4096, 1), (4096, 2), (4096, 4),
                       (4096, 8), (12288, 4), (1032, 3), (96, 4), (8, 1), (64, 8)]:
            for f32 in (False, True):
                rc = lib.check_launch(M, 97, K, S, f32)
                if rc != 0:
                    failures.append((M, K, S, f32, rc))
    assert not failures, failures[:10]


def test_line_tactic_needs_whole_line_pairs(lib):
    t = binding.tactic("line", 16, 2, 4)
    assert lib.check_launch(4, 6144, 4096, 2, tactic=t) == 0
    assert lib.check_launch(4, 6144, 4096, 2, True, tactic=t) == 0
    # K / split_k = 1984: 248 vectors, not a whole number of 64-K line pairs per wavefront
    assert lib.check_launch(4, 6144, 3968, 2, tactic=t) == binding.LOWM_ERR_UNSUPPORTED
    # more than two 16-row activation blocks, unroll other than 2, a ring past the LDS budget
    assert lib.check_launch(40, 6144, 4096, 2, tactic=t) == binding.LOWM_ERR_UNSUPPORTED
    assert lib.check_launch(4, 6144, 4096, 2, tactic=binding.tactic("line", 16, 4, 4)) == \
        binding.LOWM_ERR_UNSUPPORTED
    assert lib.check_launch(4, 6144, 4096, 2, tactic=binding.tactic("line", 64, 2, 2)) == \
        binding.LOWM_ERR_UNSUPPORTED
    assert repr(t).startswith("Tactic(line")


def test_pick_split_k(lib):
    # the measured table at its grid points (MI355X, default tactic per
    # split_k; bench.py --split-sweep)
    assert lib.pick_split_k(4, 6144, 4096) == 1
    assert lib.pick_split_k(4, 6144, 8192) == 2
    assert lib.pick_split_k(4, 768, 4096) == 4
    assert lib.pick_split_k(4, 1536, 8192) == 4
    assert lib.pick_split_k(4, 3072, 16384) == 4
    assert lib.pick_split_k(4, 12288, 4096) == 2
    assert lib.pick_split_k(8, 768, 8192) == 8
    assert lib.pick_split_k(16, 768, 4096) == 4
    assert lib.pick_split_k(16, 6144, 4096) == 1
    assert lib.pick_split_k(16, 24576, 16384) == 4
    assert lib.pick_split_k(32, 768, 16384) == 8
    assert lib.pick_split_k(32, 6144, 4096) == 1
    assert lib.pick_split_k(64, 6144, 4096) == 1
    assert lib.pick_split_k(64, 3072, 8192) == 4
    # rows: M <= 4, <= 8, <= 16, <= 32, else the M 64 measurements
    assert lib.pick_split_k(4, 768, 8192) == 4 and lib.pick_split_k(5, 768, 8192) == 8
    assert lib.pick_split_k(9, 1536, 8192) == 4 and lib.pick_split_k(8, 768, 8192) == 8
    assert lib.pick_split_k(17, 768, 8192) == 2 and lib.pick_split_k(33, 1536, 2048) == 1
    assert lib.pick_split_k(64, 768, 16384) == 8 and lib.pick_split_k(64, 768, 8192) == 1
    assert lib.pick_split_k(64, 24576, 16384) == 2 and lib.pick_split_k(64, 12288, 16384) == 1
    assert lib.pick_split_k(64, 24576, 8192) == 1
    # always a split_k the launch accepts
    for M in (1, 4, 9, 16, 33, 64):
        for N in (1, 100, 768, 2304, 6144, 100000):
            for K in (8, 64, 264, 1032, 2048, 4096, 12288, 16384, 65536):
                S = lib.pick_split_k(M, N, K)
                assert S >= 1 and (S & (S - 1)) == 0
                assert lib.check_launch(M, N, K, S) == 0, (M, N, K, S)
    t = ctypes.c_int(0)
    assert lib.lib.lowm_pick_split_k(0, 64, 256, ctypes.byref(t)) == binding.LOWM_ERR_INVALID_ARG
    assert lib.lib.lowm_pick_split_k(65, 64, 256, ctypes.byref(t)) == binding.LOWM_ERR_UNSUPPORTED
    assert lib.lib.lowm_pick_split_k(4, 64, 256, None) == binding.LOWM_ERR_INVALID_ARG


def batch_call(lib, descs, count=None, M=4, K=256, S=2, ws=FAKE_WS):
    n = len(descs) if count is None else count
    arr = (binding.GemmDesc * max(1, len(descs)))(*descs)
    return lib.lib.lowm_gemm_splitk_batched(arr if descs else None, n, M, K, S, ws, None)


def test_batched_validation(lib):
    d = binding.GemmDesc(FAKE_A, FAKE_W, FAKE_C, 64)
    assert batch_call(lib, [], count=0) == binding.LOWM_ERR_INVALID_ARG
    assert batch_call(lib, [d], count=0) == binding.LOWM_ERR_INVALID_ARG
    assert batch_call(lib, [d] * 9) == binding.LOWM_ERR_UNSUPPORTED
    assert batch_call(lib, [d, binding.GemmDesc(FAKE, 0, FAKE, 64)]) == binding.LOWM_ERR_INVALID_ARG
    assert batch_call(lib, [d, binding.GemmDesc(FAKE, FAKE, FAKE, 0)]) == binding.LOWM_ERR_INVALID_ARG
    assert batch_call(lib, [d, d], M=65) == binding.LOWM_ERR_UNSUPPORTED
    assert batch_call(lib, [d, binding.GemmDesc(FAKE, FAKE + 8, FAKE, 64)]) == \
        binding.LOWM_ERR_UNSUPPORTED
    assert batch_call(lib, [d, binding.GemmDesc(FAKE, FAKE, FAKE_ODD + 1, 64)]) == \
        binding.LOWM_ERR_UNSUPPORTED
    assert batch_call(lib, [d, d], ws=0) == binding.LOWM_ERR_WORKSPACE
    assert lib.lib.lowm_last_hip_error() == 0


def test_batched_outputs_must_not_overlap(lib):
    """Outputs of one launch must not meet each other, any operand of the
    launch or the workspace; inputs may be shared (they are only read), which
    the GPU tests exercise."""
    E = binding
    G = binding.GemmDesc
    d0 = G(FAKE_A, FAKE_W, FAKE_C, 64)
    assert batch_call(lib, [d0, G(FAKE_A, FAKE_W, FAKE_C + 256, 64)]) == E.LOWM_ERR_INVALID_ARG
    assert batch_call(lib, [d0, G(FAKE_A, FAKE_W + 0x100000, FAKE_W, 64)]) == \
        E.LOWM_ERR_INVALID_ARG                      # GEMM 1's C over GEMM 0's W
    assert batch_call(lib, [d0, G(FAKE_A + 0x100000, FAKE_W, FAKE_A, 64)]) == \
        E.LOWM_ERR_INVALID_ARG                      # GEMM 1's C over GEMM 0's A
    # the workspace is the two GEMMs' workspaces back to back: GEMM 1's C
    # just past the first one still meets the second
    ws0 = lib.workspace_bytes(4, 64, 256, 2)
    assert batch_call(lib, [d0, G(FAKE_A, FAKE_W, FAKE_WS + ws0, 64)]) == E.LOWM_ERR_INVALID_ARG
    assert lib.lib.lowm_last_hip_error() == 0


def test_batched_workspace_is_the_concatenation(lib):
    Ns = [6144, 1024, 300]
    assert lib.batched_workspace_bytes(4, Ns, 4096, 2) == sum(
        lib.workspace_bytes(4, N, 4096, 2) for N in Ns)
    assert lib.batched_workspace_bytes(4, Ns, 4096, 1) == 0
    assert lib.batched_workspace_bytes(4, [64] * 9, 4096, 2) == 0
    for N in (1, 17, 300, 6144):
        assert lib.workspace_bytes(4, N, 4096, 2) % 256 == 0


def test_check_launch_reports_validation_errors(lib):
    assert lib.check_launch(0, 64, 256, 1) == binding.LOWM_ERR_INVALID_ARG
    assert lib.check_launch(65, 64, 256, 1) == binding.LOWM_ERR_UNSUPPORTED
    assert lib.check_launch(4, 64, 260, 2) == binding.LOWM_ERR_UNSUPPORTED
    assert lib.check_launch(4, 64, 256, 2, tactic=binding.tactic("reg", 80, 4, 3)) == \
        binding.LOWM_ERR_UNSUPPORTED
    assert lib.check_launch(4, 64, 256, 2) == 0


C_ADDR, PUSH_ADDR, FLAG_ADDR = 0x10000, 0x100000, 0x200000


def push_call(lib, push=PUSH_ADDR, ld=64, flags=FLAG_ADDR, value=1, C=C_ADDR, M=4, N=64,
              K=256, S=2, ws=FAKE_WS):
    return lib.lib.lowm_gemm_splitk_push(FAKE_A, FAKE_W, C, M, N, K, S, ws, push, ld, flags,
                                         value, None, None)


def test_push_validation(lib):
    """Every case is rejected on the host, before any HIP call."""
    E = binding
    assert push_call(lib, push=0) == E.LOWM_ERR_INVALID_ARG
    assert push_call(lib, flags=0) == E.LOWM_ERR_INVALID_ARG
    assert push_call(lib, value=0) == E.LOWM_ERR_INVALID_ARG
    assert push_call(lib, ld=63) == E.LOWM_ERR_INVALID_ARG
    assert push_call(lib, push=PUSH_ADDR + 1) == E.LOWM_ERR_UNSUPPORTED
    assert push_call(lib, flags=FLAG_ADDR + 2) == E.LOWM_ERR_UNSUPPORTED
    # overlaps: C [0x10000, +4*64*2), push rows at ld 64
    assert push_call(lib, push=C_ADDR + 256) == E.LOWM_ERR_INVALID_ARG
    assert push_call(lib, flags=C_ADDR + 100) == E.LOWM_ERR_INVALID_ARG
    assert push_call(lib, flags=PUSH_ADDR + 3 * 64 * 2) == E.LOWM_ERR_INVALID_ARG
    # a wide push row pitch puts row 3 past the flags
    assert push_call(lib, ld=(FLAG_ADDR - PUSH_ADDR) // 2) == E.LOWM_ERR_INVALID_ARG
    # the GEMM's own checks still apply
    assert push_call(lib, M=65) == E.LOWM_ERR_UNSUPPORTED
    assert push_call(lib, ws=0) == E.LOWM_ERR_WORKSPACE
    # no quarter-rows tiles with the push epilogue (each row block would
    # raise the tile's flags)
    q = binding.tactic("qrows", 16, 2, 4)
    assert lib.lib.lowm_gemm_splitk_push(FAKE_A, FAKE_W, C_ADDR, 64, 64, 256, 1, 0, PUSH_ADDR, 64,
                                         FLAG_ADDR, 1, None, ctypes.byref(q)) == \
        E.LOWM_ERR_UNSUPPORTED
    assert lib.lib.lowm_last_hip_error() == 0


def test_push_wait_validation(lib):
    w = lib.lib.lowm_push_wait
    E = binding
    assert w(FLAG_ADDR, 0, 1, 10, FAKE, None) == E.LOWM_ERR_INVALID_ARG
    assert w(FLAG_ADDR, 4, 0, 10, FAKE, None) == E.LOWM_ERR_INVALID_ARG
    assert w(0, 4, 1, 10, FAKE, None) == E.LOWM_ERR_INVALID_ARG
    assert w(FLAG_ADDR, 4, 1, 10, 0, None) == E.LOWM_ERR_INVALID_ARG
    assert w(FLAG_ADDR, 4097, 1, 10, FAKE, None) == E.LOWM_ERR_UNSUPPORTED
    assert w(FLAG_ADDR, 4, 1, 10_000_001, FAKE, None) == E.LOWM_ERR_UNSUPPORTED
    assert w(FLAG_ADDR + 2, 4, 1, 10, FAKE, None) == E.LOWM_ERR_UNSUPPORTED
    assert lib.lib.lowm_last_hip_error() == 0


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """Before any HIP call: a workspace larger than the built-in scratch is
    LOWM_ERR_SCRATCH; argument errors are those of lowm_gemm_splitk."""
    fn = lib.lib.lowm_gemm_splitk_noalloc
    M, N, K, S = 64, 16384, 4096, 8
    assert lib.workspace_bytes(M, N, K, S) > binding.SCRATCH_BYTES
    assert fn(FAKE, FAKE, FAKE, M, N, K, S, None) == binding.LOWM_ERR_SCRATCH
    assert "scratch" in lib.strerror(binding.LOWM_ERR_SCRATCH)
    assert fn(None, FAKE, FAKE, 4, 64, 256, 2, None) == binding.LOWM_ERR_INVALID_ARG
    assert fn(FAKE, FAKE, FAKE, 65, 64, 256, 2, None) == binding.LOWM_ERR_UNSUPPORTED
    assert fn(FAKE, FAKE, FAKE, 4, 64, 260, 2, None) == binding.LOWM_ERR_UNSUPPORTED
    # the largest sweep shape fits
    assert lib.workspace_bytes(64, 6144, 4096, 8) <= binding.SCRATCH_BYTES


def test_workspace_status_validation(lib):
    """Before any HIP call: NULL pointers and N <= 0 are invalid arguments."""
    fn = lib.lib.lowm_workspace_status
    out = ctypes.c_int(7)
    E = binding
    assert fn(None, 64, None, ctypes.byref(out), ctypes.byref(out)) == E.LOWM_ERR_INVALID_ARG
    assert fn(FAKE, 0, None, ctypes.byref(out), ctypes.byref(out)) == E.LOWM_ERR_INVALID_ARG
    assert fn(FAKE, 64, None, None, ctypes.byref(out)) == E.LOWM_ERR_INVALID_ARG
    assert fn(FAKE, 64, None, ctypes.byref(out), None) == E.LOWM_ERR_INVALID_ARG
    assert out.value == 7
    assert lib.lib.lowm_last_hip_error() == 0


def test_quarter_tiles_built_where_lds_allows(lib):
    """Quarter tiles exist for every M, rows 16/32/64 and rings 2/3/4 whose
    four per-wavefront rings fit: 2 pieces of 1088 bytes per 16-row block of
    either operand per slot, 4 * ring slots within 160 KB of LDS, and
    (ring - 1) * loads <= 63 outstanding loads; the K slice must be whole
    64-K steps per wavefront (a multiple of 256)."""
    for M in (1, 16, 17, 32, 33, 48, 49, 64):
        for rows in (16, 32, 64):
            for ring in (2, 3, 4):
                t = binding.tactic("quarter", rows, 2, ring)
                loads = 2 * (rows // 16 + (M + 15) // 16)
                want = (ring - 1) * loads <= 63 and 4 * ring * loads * 1088 <= 160 * 1024
                rc = lib.check_launch(M, 6144, 4096, 2, tactic=t)
                assert (rc == binding.LOWM_OK) == want, (M, rows, ring, rc)
    t = binding.tactic("quarter", 32, 2, 2)
    assert lib.check_launch(32, 6144, 4096 + 128, 1, tactic=t) == binding.LOWM_ERR_UNSUPPORTED


def test_trace_buffer_bounds_the_grid(stress_lib):
    """Stress build: a launch whose grid has more workgroups than the trace
    buffer holds is refused before any HIP call (a buffer of one record
    against a grid of 16 here), and a buffer without room is rejected."""
    lib = stress_lib
    E = binding
    assert lib.lib.lowm_stress_trace(FAKE, 0) == E.LOWM_ERR_INVALID_ARG
    assert lib.lib.lowm_stress_trace(FAKE, 1) == E.LOWM_OK
    try:
        assert call(lib) == E.LOWM_ERR_INVALID_ARG          # 4 tiles -> 8, x split_k 2
        assert call(lib, M=64, N=64, S=1, tac=binding.tactic("qrows", 16, 2, 4)) == \
            E.LOWM_ERR_INVALID_ARG                          # 8 workgroups x 2 row blocks
    finally:
        assert lib.lib.lowm_stress_trace(None, 0) == E.LOWM_OK
    assert lib.lib.lowm_last_hip_error() == 0
