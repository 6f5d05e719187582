"""Properties of the host side of the C ABI over many generated shapes and
buffer layouts (no kernel is launched: every call either fails validation or
is refused for a tactic the library does not provide, before any HIP call).

- The default tactic exists for every valid shape, for both output types.
- The tile family the picker chooses does not depend on N, so a batched
  launch (picked for its narrowest GEMM) keeps each GEMM's summation order
  (the quarter-rows tiles count as quarter tiles: the same kernel and order
  over blocks of activation rows; the GPU tests check their bits).
- lowm_pick_split_k returns a split_k the library launches for that shape.
- Workspace sizes: zero without split-K, at least the counters and the fp32
  partials otherwise, and a batch's is the sum of its GEMMs'.
- The overlap rule for outputs matches a model written from the header's
  contract, on both sides (rejected and accepted layouts).
"""
from __future__ import annotations

import ctypes

import pytest
from hypothesis import HealthCheck, assume, given, settings
from hypothesis import strategies as st

import split_bf16_gemm_amd as sbg
from split_bf16_gemm_amd import binding

SETTINGS = settings(max_examples=300, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.function_scoped_fixture])
BOGUS = binding.Tactic(99, 16, 4, 2, 2)   # a tactic no build provides: refused, never launched


@pytest.fixture(scope="module")
def lib():
    return sbg.load()


@st.composite
def shapes(draw):
    """A valid (M, K, split_k): K a multiple of 8 * split_k, up to 32768."""
    M = draw(st.integers(1, 64))
    S = draw(st.sampled_from([1, 2, 3, 4, 5, 8, 16]))
    units = draw(st.integers(1, max(1, 32768 // (8 * S))))
    return M, 8 * S * units, S


# N over the whole range, with the small widths (where the rules change
# with the number of workgroups) drawn often
WIDTHS = st.one_of(st.integers(1, 8192), st.integers(1, 1 << 17))


@SETTINGS
@given(shape=shapes(), N=WIDTHS)
def test_default_tactic_exists_and_launches(lib, shape, N):
    M, K, S = shape
    t = lib.pick_tactic(M, N, K, S)
    assert t.rows in (16, 32, 48, 64) and t.waves == 4
    for f32 in (False, True):
        assert lib.check_launch(M, N, K, S, f32out=f32, tactic=t) == binding.LOWM_OK, (M, N, K, S, t)
        assert lib.check_launch(M, N, K, S, f32out=f32) == binding.LOWM_OK


@SETTINGS
@given(shape=shapes(), N1=WIDTHS, N2=WIDTHS)
def test_tile_family_does_not_depend_on_n(lib, shape, N1, N2):
    M, K, S = shape
    t1, t2 = lib.pick_tactic(M, N1, K, S), lib.pick_tactic(M, N2, K, S)
    # quarter-rows tiles run the quarter kernel on blocks of rows: one family
    family = {binding.LOWM_STAGE_QUARTER_ROWS: binding.LOWM_STAGE_QUARTER}
    assert family.get(t1.stage, t1.stage) == family.get(t2.stage, t2.stage), \
        (M, K, S, N1, t1, N2, t2)
    if t1.stage in (binding.LOWM_STAGE_REG, binding.LOWM_STAGE_LDS):
        # the register and LDS rings: one shape of ring for every N
        assert (t1.rows, t1.unroll, t1.stages) == (t2.rows, t2.unroll, t2.stages)


@SETTINGS
@given(M=st.integers(1, 64), N=WIDTHS, K=st.integers(1, 1 << 16).map(lambda k: 8 * k))
def test_picked_split_k_launches(lib, M, N, K):
    S = lib.pick_split_k(M, N, K)
    assert S in (1, 2, 4, 8)
    assert K % (8 * S) == 0
    assert lib.check_launch(M, N, K, S) == binding.LOWM_OK


@SETTINGS
@given(shape=shapes(), Ns=st.lists(st.integers(1, 1 << 16), min_size=1, max_size=8))
def test_workspace_sizes(lib, shape, Ns):
    M, K, S = shape
    singles = [lib.workspace_bytes(M, N, K, S) for N in Ns]
    for N, ws in zip(Ns, singles):
        if S == 1:
            assert ws == 0
        else:
            assert ws % 256 == 0
            assert ws >= sbg.counter_bytes(N) + 4 * S * M * N
    assert lib.batched_workspace_bytes(M, Ns, K, S) == sum(singles)


# --- the overlap rule --------------------------------------------------------
# Buffers are placed at 16-byte-aligned fake addresses inside a 1 MiB window
# well away from zero; the model below restates the header's rule: C must not
# overlap A, W or the workspace; the workspace must not overlap A or W; A and
# W may overlap each other.

BASE = 0x40000000


def span(addr, nbytes):
    return addr, addr + nbytes


def meets(a, b):
    return a[0] < b[1] and b[0] < a[1]


@st.composite
def layouts(draw):
    M = draw(st.integers(1, 8))
    N = draw(st.integers(1, 96))
    S = draw(st.sampled_from([1, 2]))
    K = 16 * draw(st.integers(1, 16))
    f32 = draw(st.booleans())
    slot = st.integers(0, (1 << 16) - 1).map(lambda i: BASE + 16 * i)
    return M, N, K, S, f32, draw(slot), draw(slot), draw(slot), draw(slot)


@SETTINGS
@given(layout=layouts())
def test_overlap_rule_matches_the_contract(lib, layout):
    M, N, K, S, f32, a, w, c, ws = layout
    A, W = span(a, 2 * M * K), span(w, 2 * N * K)
    C = span(c, (4 if f32 else 2) * M * N)
    WS = span(ws, lib.workspace_bytes(M, N, K, S)) if S > 1 else None
    bad = meets(C, A) or meets(C, W) or (
        WS is not None and (meets(C, WS) or meets(WS, A) or meets(WS, W)))
    fn = lib.lib.lowm_gemm_splitk_f32out_ex if f32 else lib.lib.lowm_gemm_splitk_ex
    rc = fn(a, w, c, M, N, K, S, ws if S > 1 else 0, None, ctypes.byref(BOGUS))
    # past validation the bogus tactic is refused before any HIP call
    assert rc == (binding.LOWM_ERR_INVALID_ARG if bad else binding.LOWM_ERR_UNSUPPORTED), layout
    assert lib.lib.lowm_last_hip_error() == 0


@st.composite
def batch_layouts(draw):
    count = draw(st.integers(2, 4))
    M = draw(st.integers(1, 8))
    K = 16 * draw(st.integers(1, 8))
    S = draw(st.sampled_from([1, 2]))
    slot = st.integers(0, (1 << 12) - 1).map(lambda i: BASE + 16 * i)
    gemms = [(draw(st.integers(1, 64)), draw(slot), draw(slot), draw(slot)) for _ in range(count)]
    return M, K, S, gemms, draw(slot)


@SETTINGS
@given(layout=batch_layouts())
def test_batched_overlaps_are_rejected(lib, layout):
    """Layouts that break the rule are rejected (the batched entry point has
    no tactic argument, so only rejected layouts are handed in)."""
    M, K, S, gemms, ws = layout
    As = [span(a, 2 * M * K) for (N, a, w, c) in gemms]
    Ws = [span(w, 2 * N * K) for (N, a, w, c) in gemms]
    Cs = [span(c, 2 * M * N) for (N, a, w, c) in gemms]
    WS = span(ws, lib.batched_workspace_bytes(M, [g[0] for g in gemms], K, S)) if S > 1 else None
    ins = As + Ws
    bad = any(meets(C, X) for C in Cs for X in ins)
    bad = bad or any(meets(Cs[i], Cs[j]) for i in range(len(Cs)) for j in range(len(Cs)) if i != j)
    if WS is not None:
        bad = bad or any(meets(WS, X) for X in ins + Cs)
    assume(bad)
    arr = (binding.GemmDesc * len(gemms))(*[binding.GemmDesc(a, w, c, N) for (N, a, w, c) in gemms])
    rc = lib.lib.lowm_gemm_splitk_batched(arr, len(gemms), M, K, S, ws if S > 1 else 0, None)
    assert rc == binding.LOWM_ERR_INVALID_ARG, layout
    assert lib.lib.lowm_last_hip_error() == 0
