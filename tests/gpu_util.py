"""Shared helpers of the GPU tests: run the HIP path, cache oracle results."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import split_bf16_gemm_amd as sbg
import workloads
from split_bf16_gemm_amd import binding


# Every bf16 output judged against the oracle: (case, elements, n_cancel,
# max_ulp), where n_cancel counts the elements that passed only through the
# cancellation rule of tests/checks.py.  Printed at the end of the session.
CANCEL_REPORT: list = []


def report(what: str, v: dict, elements: int):
    CANCEL_REPORT.append((what, elements, v["n_cancel"], v["max_ulp"]))


def say(*parts):
    """Name the case before a GPU step, flushed, so a fault can be placed."""
    print("[gpu]", *parts, file=sys.stderr, flush=True)


def device() -> torch.device:
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device")
    return torch.device("cuda:0")


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@functools.lru_cache(maxsize=64)
def inputs(wl: workloads.Workload):
    A, W = workloads.make_inputs(wl)
    return A, W


@functools.lru_cache(maxsize=64)
def oracle_result(wl: workloads.Workload):
    A, W = inputs(wl)
    return oracle.gemm(workloads.bits(A), workloads.bits(W))


VARIANTS = [("lds", 4, 2), ("lds", 4, 3),
            ("reg", 4, 2), ("reg", 8, 2), ("reg", 16, 2),
            ("line", 2, 2), ("line", 2, 3), ("line", 2, 4)]
PANEL_RINGS = (3, 4, 6)
QUARTER_RINGS = (2, 3, 4)


def all_tactics(M: int):
    """Every tactic the library may provide for M activation rows (the
    launch returns LOWM_ERR_UNSUPPORTED for those it lacks)."""
    out = []
    for rows in (16, 32):
        for stage, unroll, stages in VARIANTS:
            out.append(binding.tactic(stage, rows, unroll, stages))
    for rows in (64, 32):
        for ring in PANEL_RINGS:
            out.append(binding.tactic("panel", rows, 2, ring))
    for rows in (16, 32, 64):
        for ring in QUARTER_RINGS:
            out.append(binding.tactic("quarter", rows, 2, ring))
    return out


def quarter_built(M: int, rows: int, ring: int) -> bool:
    """Whether the build provides quarter tiles of `rows` rows and a ring of
    `ring` steps for M activation rows: each wavefront's ring slot holds 2
    pieces of 1088 bytes per 16-row block of either operand; the four rings
    must fit 160 KB of LDS and their loads the 6-bit wait counter."""
    loads = 2 * (rows // 16 + (M + 15) // 16)
    return (ring - 1) * loads <= 63 and 4 * ring * loads * 1088 <= 160 * 1024


def run(lib, A_cpu, W_cpu, split_k, f32out=False, tactic=None, workspace=None, dev=None):
    """One launch through the C ABI; returns the output as a CPU tensor.

    Returns None when the build does not provide ``tactic`` for this M."""
    dev = dev or device()
    A = A_cpu.to(dev)
    W = W_cpu.to(dev)
    M, K = A.shape
    N = W.shape[0]
    if workspace is None:
        workspace = lib.make_workspace(M, N, K, split_k, dev)
    try:
        out = lib.gemm(A, W, split_k, workspace=workspace, tactic=tactic,
                       out_dtype=torch.float32 if f32out else torch.bfloat16)
    except sbg.LowmError as e:
        if tactic is not None and e.code == binding.LOWM_ERR_UNSUPPORTED:
            return None
        raise
    torch.cuda.synchronize()
    return out.cpu()


def assert_bf16_launch(lib, A_dev, W_dev, wl, bits, tactic=None, what=""):
    """Judge a bf16 output with the rules of tests/checks.py, taking the fp32
    sibling's output (same kernel and order) for the cancellation rule."""
    import oracle
    from checks import assert_bf16, assert_fp32
    C, S = oracle_result(wl)
    ws = lib.make_workspace(wl.M, wl.N, wl.K, wl.split_k, A_dev.device)
    c32 = lib.gemm(A_dev, W_dev, wl.split_k, workspace=ws, tactic=tactic,
                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    c32 = c32.cpu().numpy()
    assert_fp32(c32, C, S, what=what)
    assert np.array_equal(bits, oracle.round_bf16(c32.astype(np.float64))), \
        f"{what}: bf16 output is not RNE of the fp32 sibling"
    v = assert_bf16(bits, C, S, wl.K, oracle.default(), c32, what=what)
    report(what or wl.name, v, C.size)
    return v
