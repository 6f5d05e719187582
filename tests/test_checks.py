"""The parity comparators catch the mistakes a split-K GEMM can make.

Mistakes are planted in oracle results on the CPU (never in a GPU kernel): a
missing K slice (one rank's partial never added), swapped output rows, a bf16
value two ulps off, a stale partial from other inputs.  Correct alternatives
(fp32 rounding of the oracle, the two rank partials folded in either order)
must pass.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from checks import assert_bf16, assert_fp32, assert_exact_integer, bf16_ord, bf16_verdict


@pytest.fixture(scope="module")
def case():
    orc = oracle.default()
    wl = workloads.Workload("checks", 4, 256, 4096, 2, seed_a=31, seed_w=32)
    A, W = workloads.make_inputs(wl)
    a, w = workloads.bits(A), workloads.bits(W)
    C, S = orc.gemm(a, w)
    half = wl.K // 2
    P0, _ = orc.gemm(a[:, :half].copy(), w[:, :half].copy())
    P1, _ = orc.gemm(a[:, half:].copy(), w[:, half:].copy())
    return orc, wl, a, w, C, S, P0, P1


def test_correct_fp32_and_bf16_pass(case):
    orc, wl, a, w, C, S, P0, P1 = case
    c32 = C.astype(np.float32)
    assert_fp32(c32, C, S)
    v = assert_bf16(orc.round_bf16(c32.astype(np.float64)), C, S, wl.K, orc, c32)
    assert v["max_ulp"] <= 1


def test_both_fold_orders_pass(case):
    orc, wl, a, w, C, S, P0, P1 = case
    for c32 in ((P0.astype(np.float32) + P1.astype(np.float32)),
                (P1.astype(np.float32) + P0.astype(np.float32))):
        assert_fp32(c32, C, S)
        assert_bf16(orc.round_bf16(c32.astype(np.float64)), C, S, wl.K, orc, c32)


def test_missing_slice_fails(case):
    orc, wl, a, w, C, S, P0, P1 = case
    c32 = P0.astype(np.float32)         # rank 1's partial never added
    with pytest.raises(AssertionError):
        assert_fp32(c32, C, S)
    with pytest.raises(AssertionError):
        assert_bf16(orc.round_bf16(c32.astype(np.float64)), C, S, wl.K, orc, c32)


def test_swapped_rows_fail(case):
    orc, wl, a, w, C, S, P0, P1 = case
    c32 = C.astype(np.float32)[[1, 0, 2, 3]]
    with pytest.raises(AssertionError):
        assert_fp32(c32, C, S)


def test_stale_partial_fails(case):
    # the second rank's slot still holds a partial of different inputs
    orc, wl, a, w, C, S, P0, P1 = case
    rng = np.random.default_rng(0)
    stale = P1[:, rng.permutation(P1.shape[1])]
    c32 = (P0 + stale).astype(np.float32)
    with pytest.raises(AssertionError):
        assert_fp32(c32, C, S)


def test_one_ulp_passes_two_ulps_fail(case):
    orc, wl, a, w, C, S, P0, P1 = case
    ref = orc.round_bf16(C)
    big = np.unravel_index(np.argmax(np.abs(C)), C.shape)
    one = ref.copy()
    one[big] = np.uint16(int(one[big]) + 1)
    assert bf16_verdict(one, C, S, wl.K, orc)["n_fail"] == 0
    two = ref.copy()
    two[big] = np.uint16(int(two[big]) + 2)
    with pytest.raises(AssertionError):
        assert_bf16(two, C, S, wl.K, orc, C.astype(np.float32))


def test_ord_is_monotone_across_zero():
    bits = np.array([0x8001, 0x8000, 0x0000, 0x0001, 0x3F80], dtype=np.uint16)
    o = bf16_ord(bits)
    assert list(o) == [-1, 0, 0, 1, 0x3F80]


def test_integer_exactness_check():
    orc = oracle.default()
    C = np.array([[3.0, -7.0, 300.0]])
    good32 = C.astype(np.float32)
    good16 = orc.round_bf16(C)
    assert_exact_integer(good32, good16, C, orc)
    bad32 = good32.copy()
    bad32[0, 1] = np.nextafter(np.float32(-7.0), np.float32(0))
    with pytest.raises(AssertionError):
        assert_exact_integer(bad32, good16, C, orc)
    bad16 = good16.copy()
    bad16[0, 2] ^= 1
    with pytest.raises(AssertionError):
        assert_exact_integer(good32, bad16, C, orc)
