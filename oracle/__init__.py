"""Host-only fp64 oracle for the low-M split-K bf16 GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``split_bf16_gemm_amd``) never imports, links or calls it, and the two share no
code: the arithmetic lives in ``oracle.c``, compiled here with gcc.

What the oracle computes is the plain definition of the product the split-K
kernel reaches up to rounding order, C = A * W^T with A [M, K] and W [N, K]
row-major bf16 (TensorRT-LLM PR "Fix two synchronization gaps in the MiniMax M3
low-M split-K GEMM", Description item 2 and Hardware verification), summed in
fp64 in ascending k, together with S = |A| * |W|^T, the scale of every error
bound.  Rounding to bf16 is round-to-nearest-even taken directly from fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "oracle.c"
LIBRARY = HERE / "liboracle.so"

# -O2 without fast-math and without contraction: each fp64 operation is one
# IEEE operation, in the order the source writes it.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra"]


def build(source: Path = SOURCE, output: Path = LIBRARY) -> Path:
    """Compile ``source`` into the shared library ``output`` with gcc."""
    tmp = Path(str(output) + f".tmp{os.getpid()}")
    cmd = ["gcc", *CFLAGS, "-o", str(tmp), str(source), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Path | str):
        lib = ctypes.CDLL(str(path))
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_bf16_to_f64_array.argtypes = [_u16p, _f64p, _i64]
        lib.oracle_bf16_to_f64_array.restype = None
        lib.oracle_round_bf16_array.argtypes = [_f64p, _u16p, _i64]
        lib.oracle_round_bf16_array.restype = None
        lib.oracle_gemm_f64_cols.argtypes = [_u16p, _u16p, _i64, _i64, _i64,
                                             _i64, _i64, _f64p, _f64p]
        lib.oracle_gemm_f64_cols.restype = None
        self._lib = lib
        self.path = Path(path)

    # -- scalar / element-wise -------------------------------------------
    def bf16_to_f64(self, bits) -> np.ndarray:
        """Exact value of each bf16 bit pattern (uint16 array)."""
        b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
        out = np.empty(b.shape, dtype=np.float64)
        self._lib.oracle_bf16_to_f64_array(b.ctypes.data_as(_u16p),
                                           out.ctypes.data_as(_f64p), b.size)
        return out

    def round_bf16(self, x) -> np.ndarray:
        """Nearest bf16 bit pattern (ties to even) of each fp64 value."""
        v = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(v.shape, dtype=np.uint16)
        self._lib.oracle_round_bf16_array(v.ctypes.data_as(_f64p),
                                          out.ctypes.data_as(_u16p), v.size)
        return out

    # -- the product -------------------------------------------------------
    def gemm_cols(self, a_bits, w_bits, n_begin: int, n_end: int):
        """Columns [n_begin, n_end) of C = A W^T and S = |A| |W|^T (fp64)."""
        a = np.ascontiguousarray(np.asarray(a_bits, dtype=np.uint16))
        w = np.ascontiguousarray(np.asarray(w_bits, dtype=np.uint16))
        if a.ndim != 2 or w.ndim != 2 or a.shape[1] != w.shape[1]:
            raise ValueError(f"bad operand shapes {a.shape} and {w.shape}")
        M, K = a.shape
        N = w.shape[0]
        if not 0 <= n_begin <= n_end <= N:
            raise ValueError(f"bad column range [{n_begin}, {n_end}) for N={N}")
        width = n_end - n_begin
        C = np.zeros((M, width), dtype=np.float64)
        S = np.zeros((M, width), dtype=np.float64)
        self._lib.oracle_gemm_f64_cols(a.ctypes.data_as(_u16p),
                                       w.ctypes.data_as(_u16p), M, N, K,
                                       n_begin, n_end,
                                       C.ctypes.data_as(_f64p),
                                       S.ctypes.data_as(_f64p))
        return C, S

    def gemm(self, a_bits, w_bits):
        """C = A W^T and S = |A| |W|^T over all columns (fp64)."""
        w = np.asarray(w_bits)
        return self.gemm_cols(a_bits, w_bits, 0, w.shape[0])


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``oracle.c``; compiled on first use if absent."""
    global _default
    if _default is None:
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
            build()
        _default = Oracle(LIBRARY)
    return _default


def bf16_to_f64(bits):
    return default().bf16_to_f64(bits)


def round_bf16(x):
    return default().round_bf16(x)


def gemm(a_bits, w_bits):
    return default().gemm(a_bits, w_bits)


def gemm_cols(a_bits, w_bits, n_begin, n_end):
    return default().gemm_cols(a_bits, w_bits, n_begin, n_end)
