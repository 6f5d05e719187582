"""Operands past 2^31 elements: W of 139,264 x 16,384 bf16 (2.28e9 elements,
4.6 GB), so every weight-row offset beyond row 131,072 exceeds 32 bits.  The
line-pair, quarter and panel tiles each run the whole product; sampled column
ranges (the first, those across row 131,072, the last) are judged against the
oracle on the same W rows, copied back to the host."""
from __future__ import annotations

import pytest
import torch

import oracle
import split_bf16_gemm_amd as sbg
import workloads
from checks import assert_bf16, assert_fp32
from gpu_util import device, report, say, to_bits

pytestmark = pytest.mark.gpu

N_BIG, K_BIG = 139264, 16384
assert N_BIG * K_BIG > 2 ** 31
SAMPLES = [(0, 16), (131072 - 16, 131072 + 16), (N_BIG - 16, N_BIG)]


@pytest.fixture(scope="module")
def big_w():
    dev = device()
    say("large W", N_BIG, K_BIG)
    W = workloads.make_large_w(N_BIG, K_BIG, seed=5150, device=dev)
    torch.cuda.synchronize()
    yield W
    del W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,S", [(4, 2), (4, 1), (64, 2)])
def test_operands_past_two_to_the_31_elements(big_w, M, S):
    lib = sbg.load()
    dev = device()
    wl = workloads.Workload(f"large_m{M}_s{S}", M, 1, K_BIG, S, seed_a=5200 + M)
    A_cpu, _ = workloads.make_inputs(wl)
    A = A_cpu.to(dev)
    ws = lib.make_workspace(M, N_BIG, K_BIG, S, dev)
    say("large", M, N_BIG, K_BIG, S, lib.pick_tactic(M, N_BIG, K_BIG, S))
    c32 = lib.gemm(A, big_w, S, workspace=ws, out_dtype=torch.float32)
    c16 = lib.gemm(A, big_w, S, workspace=ws)
    torch.cuda.synchronize()
    a_bits = workloads.bits(A_cpu)
    for n0, n1 in SAMPLES:
        w_bits = workloads.bits(big_w[n0:n1].cpu())
        C, Sc = oracle.gemm_cols(a_bits, w_bits, 0, n1 - n0)
        what = f"large M {M} split_k {S} columns {n0}..{n1}"
        got32 = c32[:, n0:n1].cpu().numpy()
        assert_fp32(got32, C, Sc, what=what)
        b16 = to_bits(c16[:, n0:n1])
        v = assert_bf16(b16, C, Sc, K_BIG, oracle.default(), got32, what=what)
        report(what, v, C.size)
    if ws is not None:
        assert not ws.cpu().numpy().any(), "the workspace was left non-zero"
