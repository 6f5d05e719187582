"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an oracle instance and raises AssertionError when it is
wrong.  Sources of truth:
  * the IEEE-754 meaning of bf16 (all 65536 patterns against torch's decode)
    and hand-derived rounding cases (tests/golden/bf16_rounding.txt);
  * a hand-computed product (tests/golden/tiny_gemm.txt);
  * the integer closed form of the Triton issue "warpgroup_mma_wait does not
    properly synchronize across warpgroups" (Describe the bug): all-ones times
    integers in [-3, 3], expected value the column sums, exact below 2^24;
  * exact integer products (numpy int64), exact rational sums on tiny shapes
    (fractions.Fraction, an independent round-to-nearest-even written here),
    torch's CPU fp64 matmul, and the permutation invariance of the product.
``test_mutants_are_caught`` plants plausible mistakes in a copy of the
oracle's C source and checks that every one of them fails at least one pin.
"""
from __future__ import annotations

from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from checks import U_FP64, gamma
import workloads

GOLDEN = Path(__file__).resolve().parent / "golden"


# --------------------------------------------------------------------------
# independent helpers (no oracle code)
# --------------------------------------------------------------------------
def torch_bf16_decode(bits_u16: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(bits_u16.astype(np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def torch_round_bf16_from_f32(x_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fraction_rne_bf16(x: Fraction) -> int:
    """Round an exact rational to the nearest bf16 pattern, ties to even."""
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    if e < -126:
        q = round(a / Fraction(2) ** -133)   # Fraction.__round__: half to even
        return sign | q
    q = round(a / Fraction(2) ** (e - 7))    # in [128, 256]
    if q == 256:
        q, e = 128, e + 1
    if e + 127 >= 255:
        return sign | 0x7F80
    return sign | ((e + 127) << 7) | (q - 128)


def bf16_fraction(bits: int) -> Fraction:
    """Exact value of a finite bf16 pattern, from the field layout."""
    s = -1 if bits & 0x8000 else 1
    ex = (bits >> 7) & 0xFF
    fr = bits & 0x7F
    if ex == 0:
        return s * Fraction(fr) * Fraction(2) ** (-133)
    return s * Fraction(128 + fr) * Fraction(2) ** (ex - 134)


def random_bf16_bits(rng: np.random.Generator, shape, scale=1.0) -> np.ndarray:
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch_round_bf16_from_f32(x)


def read_rounding_cases():
    rows = []
    for line in (GOLDEN / "bf16_rounding.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        tok = line.split()
        x = {"inf": np.inf, "-inf": -np.inf, "nan": np.nan}.get(tok[0])
        if x is None:
            x = float.fromhex(tok[0])
        rows.append((x, int(tok[1], 16), " ".join(tok[2:])))
    return rows


def read_tiny_gemm():
    d = {}
    for line in (GOLDEN / "tiny_gemm.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        key, *vals = line.split()
        d[key] = vals
    M, N, K = int(d["M"][0]), int(d["N"][0]), int(d["K"][0])
    A = np.array([int(v, 16) for v in d["A"]], dtype=np.uint16).reshape(M, K)
    W = np.array([int(v, 16) for v in d["W"]], dtype=np.uint16).reshape(N, K)
    C = np.array([float(v) for v in d["C"]]).reshape(M, N)
    S = np.array([float(v) for v in d["S"]]).reshape(M, N)
    Cb = np.array([int(v, 16) for v in d["C_bf16"]], dtype=np.uint16).reshape(M, N)
    return A, W, C, S, Cb


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def pin_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_f64(bits)
    want = torch_bf16_decode(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns decode differently"
    assert np.array_equal(got[~nan], want[~nan]), "bf16 decode differs from torch"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), "sign of zero"


def pin_round_golden(orc):
    for x, want, why in read_rounding_cases():
        got = int(orc.round_bf16(np.array([x]))[0])
        assert got == want, f"round_bf16({x!r}) = {got:#06x}, want {want:#06x} ({why})"


def pin_round_matches_torch_on_fp32(orc):
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # force exact ties: lower half exactly 0x8000, both parities above it
    raw[:20000] = (raw[:20000] & 0xFFFF0000) | 0x8000
    x32 = raw.view(np.float32)
    finite = np.isfinite(x32)
    x32 = x32[finite]
    got = orc.round_bf16(x32.astype(np.float64))
    want = torch_round_bf16_from_f32(x32)
    assert np.array_equal(got, want), "RNE disagrees with torch's fp32->bf16 cast"


def pin_tiny_gemm_golden(orc):
    A, W, C, S, Cb = read_tiny_gemm()
    c, s = orc.gemm(A, W)
    assert c.shape == C.shape and np.array_equal(c, C), f"C {c} != {C}"
    assert np.array_equal(s, S), f"S {s} != {S}"
    assert np.array_equal(orc.round_bf16(c), Cb)


def pin_closed_form(orc):
    wl = workloads.INT_EXACT
    A, W = workloads.make_inputs(wl)
    a, w = workloads.bits(A), workloads.bits(W)
    C, S = orc.gemm(a, w)
    w_int = W.to(torch.int64).numpy()
    col = w_int.sum(axis=1)                      # sum_k W[n, k]
    assert np.abs(col).max() < 2 ** 24
    assert np.array_equal(C, np.broadcast_to(col[None, :], C.shape).astype(np.float64))
    assert np.array_equal(S, np.broadcast_to(np.abs(w_int).sum(axis=1)[None, :],
                                             S.shape).astype(np.float64))


def pin_integer_matmul(orc):
    for (M, N, K, seed) in [(3, 37, 100, 11), (5, 16, 64, 12), (1, 9, 33, 13)]:
        wl = workloads.Workload("int", M, N, K, 1, kind="int_both",
                                seed_a=seed, seed_w=seed + 100)
        A, W = workloads.make_inputs(wl)
        a_i = A.to(torch.int64).numpy()
        w_i = W.to(torch.int64).numpy()
        C, S = orc.gemm(workloads.bits(A), workloads.bits(W))
        assert np.array_equal(C, (a_i @ w_i.T).astype(np.float64)), (M, N, K)
        assert np.array_equal(S, (np.abs(a_i) @ np.abs(w_i).T).astype(np.float64))


def pin_bruteforce_fraction(orc):
    rng = np.random.default_rng(3)
    for trial in range(6):
        M = int(rng.integers(1, 5))
        N = int(rng.integers(1, 18))
        K = int(rng.integers(1, 65))
        a = random_bf16_bits(rng, (M, K))
        w = random_bf16_bits(rng, (N, K), scale=0.02 if trial % 2 else 3.0)
        C, S = orc.gemm(a, w)
        got16 = orc.round_bf16(C)
        af = [[bf16_fraction(int(v)) for v in row] for row in a]
        wf = [[bf16_fraction(int(v)) for v in row] for row in w]
        bound = gamma(K, U_FP64)
        for m in range(M):
            for n in range(N):
                exact = sum((af[m][k] * wf[n][k] for k in range(K)), Fraction(0))
                mag = sum((abs(af[m][k] * wf[n][k]) for k in range(K)), Fraction(0))
                assert float(mag) == S[m, n] or abs(Fraction(S[m, n]) - mag) <= bound * mag
                err = abs(Fraction(C[m, n]) - exact)
                assert err <= bound * mag, (trial, m, n, float(err), float(mag))
                want16 = fraction_rne_bf16(exact)
                if int(got16[m, n]) != want16:
                    # only allowed when the exact value sits within fp64 error
                    # of a bf16 rounding boundary
                    lo = bf16_fraction(min(want16, int(got16[m, n])) & 0xFFFF)
                    assert err > 0, (trial, m, n, hex(int(got16[m, n])), hex(want16))
                    assert abs(abs(exact) - abs(lo)) <= bound * mag * 2 ** 9


def pin_torch_fp64(orc):
    rng = np.random.default_rng(5)
    a = random_bf16_bits(rng, (4, 1024))
    w = random_bf16_bits(rng, (96, 1024), scale=0.02)
    C, S = orc.gemm(a, w)
    ta = torch.from_numpy(orc_free_decode(a))
    tw = torch.from_numpy(orc_free_decode(w))
    ref = (ta @ tw.T).numpy()
    assert np.all(np.abs(C - ref) <= 1e-12 * S)


def orc_free_decode(bits):
    return torch_bf16_decode(bits)


def pin_cols_consistent(orc):
    wl = workloads.Workload("int", 3, 40, 96, 1, kind="int_both", seed_a=21, seed_w=22)
    A, W = workloads.make_inputs(wl)
    a_i = A.to(torch.int64).numpy()
    w_i = W.to(torch.int64).numpy()
    full = (a_i @ w_i.T).astype(np.float64)
    for lo, hi in [(0, 40), (5, 23), (39, 40), (7, 7)]:
        C, S = orc.gemm_cols(workloads.bits(A), workloads.bits(W), lo, hi)
        assert C.shape == (3, hi - lo)
        assert np.array_equal(C, full[:, lo:hi]), (lo, hi)


def pin_row_permutation(orc):
    rng = np.random.default_rng(9)
    a = random_bf16_bits(rng, (4, 200))
    w = random_bf16_bits(rng, (33, 200), scale=0.02)
    perm = rng.permutation(33)
    C, _ = orc.gemm(a, w)
    Cp, _ = orc.gemm(a, w[perm])
    assert np.array_equal(Cp, C[:, perm])


PINS = [pin_decode_all_patterns, pin_round_golden, pin_round_matches_torch_on_fp32,
        pin_tiny_gemm_golden, pin_closed_form, pin_integer_matmul,
        pin_bruteforce_fraction, pin_torch_fp64, pin_cols_consistent,
        pin_row_permutation]


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_fraction_rne_self_check():
    # the independent Fraction rounding agrees with the hand-derived table
    for x, want, why in read_rounding_cases():
        if np.isfinite(x) and not (x == 0 and np.signbit(x)):  # no -0 in Fraction
            assert fraction_rne_bf16(Fraction(x)) == want, (x, why)


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin.  The mutants run
# in this process, so every one of them keeps all accesses inside the
# buffers the pins pass (a wrong index that left them would corrupt the heap).
# --------------------------------------------------------------------------
MUTANTS = {
    "drop_last_k": ("for (int64_t k = 0; k < K; ++k) {\n                acc",
                    "for (int64_t k = 0; k < K - 1; ++k) {\n                acc"),
    "transposed_w": ("w[k] = oracle_bf16_to_f64(W[n * K + k]);",
                     "w[k] = oracle_bf16_to_f64(W[k * N + n]);"),
    "wrong_sign": ("acc += a[m * K + k] * w[k];", "acc -= a[m * K + k] * w[k];"),
    "wrong_row": ("acc += a[m * K + k] * w[k];", "acc += a[((m + 1) % M) * K + k] * w[k];"),
    "bias_off_by_one": ("expo - 127 - 7", "expo - 126 - 7"),
    "subnormal_implicit_bit": ("mag = ldexp((double)frac, -126 - 7);",
                               "mag = ldexp((double)(128 + frac), -126 - 7);"),
    "ties_away": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "truncate": ("if (rem > 0.5) return fl + 1.0;", "if (rem > 2.0) return fl + 1.0;"),
    "double_rounding": ("uint16_t sign = signbit(x) ? 0x8000u : 0u;",
                        "x = (double)(float)x;\n    uint16_t sign = signbit(x) ? 0x8000u : 0u;"),
    "signed_scale": ("mag += fabs(a[m * K + k]) * fabs(w[k]);", "mag += a[m * K + k] * w[k];"),
    "column_order": ("C[m * width + (n - n_begin)] = acc;", "C[m * width + (n_end - 1 - n)] = acc;"),
    "no_overflow": ("if (biased >= 255) return (uint16_t)(sign | 0x7F80u);", ""),
}


def test_mutants_are_caught(tmp_path):
    src = oracle.SOURCE.read_text()
    survivors = []
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation site for {name} not unique/present"
        mutated = src.replace(old, new)
        c_path = tmp_path / f"{name}.c"
        so_path = tmp_path / f"lib{name}.so"
        c_path.write_text(mutated)
        oracle.build(c_path, so_path)
        m = oracle.Oracle(so_path)
        caught = []
        for pin in PINS:
            try:
                pin(m)
            except (AssertionError, ValueError, IndexError):
                caught.append(pin.__name__)
        if not caught:
            survivors.append(name)
    assert not survivors, f"mutants not caught by any pin: {survivors}"
