"""Comparators between a GEMM result and the fp64 oracle (test infrastructure).

The bars, from the statement of the problem:
  * integer-valued inputs: every partial sum is an integer below 2^24, so the
    fp32 output must equal the oracle exactly and the bf16 output must be the
    oracle's value rounded to nearest-even, bit for bit (Triton issue
    "warpgroup_mma_wait does not properly synchronize across warpgroups",
    Describe the bug: the closed form and its 2^24 bound);
  * random inputs: the fp32 output within 1e-3 * sum_k |a||w| of the oracle,
    and the bf16 output within one ulp of the oracle's rounded value;
  * the bf16 output is compared after the same round-to-nearest-even the
    TensorRT-LLM PR "Fix two synchronization gaps in the MiniMax M3 low-M
    split-K GEMM" (Hardware verification) applies to its fp32 product.

One ulp is measured on the monotone integer line of bf16 patterns (sign and
magnitude folded, +0 = -0), so it holds across binade boundaries and zero.
Where cancellation makes |C| tiny, a correct fp32 sum can round to a bf16
several ulps from RNE(C): such an element passes only if its fp32 value lies
inside the a-priori bound gamma_K * sum|a||w| of any fp32 summation order and
its bf16 value is exactly RNE of that fp32 value.  These elements are counted.
"""
from __future__ import annotations

import numpy as np

U_FP32 = 2.0 ** -24
U_FP64 = 2.0 ** -53


def gamma(n: int, u: float = U_FP32) -> float:
    """Higham's gamma_n = n u / (1 - n u): the relative bound of an n-term sum."""
    return n * u / (1.0 - n * u)


def bf16_ord(bits) -> np.ndarray:
    """Map bf16 bit patterns to integers that increase with the value."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def fp32_within(c32, C, S, rel: float = 1e-3) -> np.ndarray:
    """Element-wise |c32 - C| <= rel * S."""
    c = np.asarray(c32, dtype=np.float64)
    return np.abs(c - C) <= rel * S


def bf16_verdict(c16_bits, C, S, K: int, orc, c32=None) -> dict:
    """Judge a bf16 output against the oracle (C, S).

    Returns a dict with the element-wise pass mask ``ok``, ``n_fail``,
    ``max_ulp`` (distance to RNE(C) in bf16 ulps) and ``n_cancel`` (elements
    that passed only through the cancellation rule above)."""
    c16 = np.asarray(c16_bits, dtype=np.uint16)
    ref = orc.round_bf16(C)
    dist = np.abs(bf16_ord(c16) - bf16_ord(ref))
    ok = dist <= 1
    n_cancel = 0
    if c32 is not None:
        c32 = np.asarray(c32, dtype=np.float32)
        far = ~ok
        if far.any():
            inside = np.abs(c32.astype(np.float64) - C) <= gamma(K) * S
            same = orc.round_bf16(c32.astype(np.float64)) == c16
            rescue = far & inside & same
            n_cancel = int(rescue.sum())
            ok = ok | rescue
    return {"ok": ok, "n_fail": int((~ok).sum()), "max_ulp": int(dist.max(initial=0)),
            "n_cancel": n_cancel}


def assert_fp32(c32, C, S, rel: float = 1e-3, what: str = ""):
    ok = fp32_within(c32, C, S, rel)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(
            f"{what}: {len(bad)} fp32 elements outside {rel} * sum|a||w|; "
            f"first at {i}: got {float(np.asarray(c32)[i])!r}, oracle {C[i]!r}, "
            f"scale {S[i]!r}")


def assert_bf16(c16_bits, C, S, K: int, orc, c32=None, what: str = ""):
    v = bf16_verdict(c16_bits, C, S, K, orc, c32)
    if v["n_fail"]:
        bad = np.argwhere(~v["ok"])
        i = tuple(bad[0])
        raise AssertionError(
            f"{what}: {v['n_fail']} bf16 elements beyond 1 ulp of RNE(oracle); "
            f"first at {i}: got {int(np.asarray(c16_bits)[i]):#06x}, "
            f"oracle {C[i]!r} -> {int(orc.round_bf16(np.array([C[i]]))[0]):#06x}")
    return v


def assert_exact_integer(c32, c16_bits, C, orc, what: str = ""):
    """Integer-valued inputs: fp32 equal to the oracle, bf16 = RNE(oracle)."""
    assert np.all(C == np.round(C)), f"{what}: oracle result is not integral"
    assert np.abs(C).max(initial=0) < 2 ** 24, f"{what}: |C| reaches 2^24"
    if c32 is not None:
        c = np.asarray(c32, dtype=np.float64)
        n_bad = int((c != C).sum())
        assert n_bad == 0, f"{what}: {n_bad} fp32 elements differ from the exact sum"
    if c16_bits is not None:
        ref = orc.round_bf16(C)
        n_bad = int((np.asarray(c16_bits, dtype=np.uint16) != ref).sum())
        assert n_bad == 0, f"{what}: {n_bad} bf16 elements differ from RNE(exact sum)"
