"""Push epilogue: each output tile's owner also writes the bf16 tile into a
caller-given exchange buffer and then sets one flag per 16 output columns.

Checked here: C and the pushed copy are each judged against the fp64 oracle
(the bars of tests/checks.py) and are bit-identical to each other and to the
plain launch's output; the copy lands exactly in the [M, N] window of a wider
strided buffer and nowhere else, each flag of the GEMM holds the caller's
value and the flags after them are untouched; a consumer that waits for the
flags on a second stream while the GEMM runs sees every flag and the final
values, which are judged against the oracle too; the wait gives up, bounded,
on flags that no launch sets."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import split_bf16_gemm_amd as sbg
import workloads
from gpu_util import assert_bf16_launch, device, inputs, say, to_bits
from split_bf16_gemm_amd import binding

pytestmark = pytest.mark.gpu

SENTINEL = -1          # 0xFFFF in every bf16 slot, all bits in every flag slot

CASES = [  # M, N, K, split_k
    (4, 6144, 4096, 2),
    (4, 300, 2048, 1),
    (4, 300, 2048, 4),
    (20, 520, 2048, 2),
    (1, 2304, 12288, 4),
]

TACTICS = [None, ("reg", 16, 4, 2), ("lds", 16, 4, 2), ("reg", 32, 4, 2)]
# panel tiles exist for 17..64 activation rows only
PANEL_CASES = [(20, 520, 2048, 2), (64, 1000, 4096, 4), (33, 6144, 4096, 1)]
# 33..64 rows without split-K: the push epilogue's own tile choice (never the
# quarter-rows tiles, whose row blocks would each raise a tile's flags)
PAIRS = ([(c, t) for c in CASES for t in TACTICS] +
         [(c, ("panel", 64, 2, 4)) for c in PANEL_CASES] +
         [(c, ("quarter", 32, 2, 3)) for c in CASES] +
         [((64, 1000, 4096, 4), ("quarter", 64, 2, 2))] +
         [((64, 2000, 4096, 1), None), ((40, 3000, 2048, 1), None)])


def window(M, N, dev, off=24, extra=40):
    ld = off + N + extra
    big = torch.full((M, ld), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    return big, big[:, off:off + N], off


@pytest.mark.parametrize("case,tac", PAIRS, ids=lambda x: (
    "x".join(map(str, x)) if isinstance(x, tuple) and isinstance(x[0], int)
    else "default" if x is None else ":".join(map(str, x))))
def test_push_copy_window_and_flags(case, tac):
    M, N, K, S = case
    lib = sbg.load()
    dev = device()
    wl = workloads.Workload(f"push_m{M}_n{N}_k{K}_s{S}", M, N, K, S, seed_a=31, seed_w=32)
    A, W = (t.to(dev) for t in inputs(wl))
    tactic = None if tac is None else binding.tactic(*tac)
    nflags = (N + 15) // 16
    flags = torch.full((nflags + 8,), SENTINEL, dtype=torch.int32, device=dev)
    flags[:nflags] = 0
    big, win, off = window(M, N, dev)
    ws = lib.make_workspace(M, N, K, S, dev)
    say("push", M, N, K, S, tac)
    C = lib.gemm_push(A, W, S, win, flags, 7, workspace=ws, tactic=tactic)
    torch.cuda.synchronize()
    plain = lib.gemm(A, W, S, workspace=ws, tactic=tactic)
    torch.cuda.synchronize()
    c = to_bits(C)
    assert np.array_equal(c, to_bits(plain)), "C of the push launch differs from the plain launch"
    b = to_bits(big)
    assert np.array_equal(b[:, off:off + N], c), "pushed copy differs from C"
    what = f"push {M}x{N}x{K} s{S} {tac}"
    assert_bf16_launch(lib, A, W, wl, c, tactic=tactic, what=what + ": C")
    assert_bf16_launch(lib, A, W, wl, np.ascontiguousarray(b[:, off:off + N]), tactic=tactic,
                       what=what + ": pushed copy")
    outside = np.ones(b.shape, dtype=bool)
    outside[:, off:off + N] = False
    assert (b[outside] == 0xFFFF).all(), "the push wrote outside its [M, N] window"
    f = flags.cpu().numpy()
    assert (f[:nflags] == 7).all(), "a flag of the GEMM was not set"
    assert (f[nflags:] == SENTINEL).all(), "a flag past the GEMM's columns was written"
    if ws is not None:
        assert not ws.cpu().numpy().any(), "the workspace was left non-zero"


def test_push_consumer_waits_on_another_stream():
    """The wait is enqueued first on a second stream; it must see every flag
    raised by the GEMM that runs after it on the current stream, and the data
    it copies afterwards must be the final output."""
    lib = sbg.load()
    dev = device()
    M, N, K, S = 4, 6144, 4096, 2
    wl = workloads.Workload("push_consumer", M, N, K, S, seed_a=41, seed_w=42)
    A, W = (t.to(dev) for t in inputs(wl))
    nflags = (N + 15) // 16
    flags = torch.zeros(nflags, dtype=torch.int32, device=dev)
    missing = torch.full((1,), -1, dtype=torch.int32, device=dev)
    big, win, _ = window(M, N, dev)
    got = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = lib.make_workspace(M, N, K, S, dev)
    consumer = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    say("push consumer wait + producer")
    lib.push_wait(flags, nflags, 3, 2_000_000, missing, stream=consumer)
    with torch.cuda.stream(consumer):
        got.copy_(win)
    C = lib.gemm_push(A, W, S, win, flags, 3, workspace=ws)
    torch.cuda.synchronize()
    assert int(missing.item()) == 0, f"the consumer timed out with {int(missing.item())} flags unseen"
    assert np.array_equal(to_bits(got), to_bits(C)), "the consumer read values before the final ones"
    assert_bf16_launch(lib, A, W, wl, to_bits(got), what="push consumer's copy")


def test_push_wait_times_out_on_flags_never_set():
    lib = sbg.load()
    dev = device()
    flags = torch.zeros(100, dtype=torch.int32, device=dev)
    flags[::3] = 5
    missing = torch.full((1,), -1, dtype=torch.int32, device=dev)
    say("push wait timeout")
    lib.push_wait(flags, 100, 5, 2000, missing)
    torch.cuda.synchronize()
    assert int(missing.item()) == 100 - 34
    # more flags than the tensor holds: refused before any launch
    with pytest.raises(ValueError):
        lib.push_wait(flags, 101, 5, 2000, missing)
    with pytest.raises(ValueError):
        lib.push_wait(flags[::2], 10, 5, 2000, missing)


def test_push_flag_value_per_call():
    """Two launches on the same flags with different values, no reset between."""
    lib = sbg.load()
    dev = device()
    M, N, K, S = 4, 1000, 2048, 2
    wl = workloads.Workload("push_twice", M, N, K, S, seed_a=51, seed_w=52)
    A, W = (t.to(dev) for t in inputs(wl))
    nflags = (N + 15) // 16
    flags = torch.zeros(nflags, dtype=torch.int32, device=dev)
    dst = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = lib.make_workspace(M, N, K, S, dev)
    missing = torch.full((1,), -1, dtype=torch.int32, device=dev)
    say("push twice")
    for value in (1, 2):
        C = lib.gemm_push(A, W, S, dst, flags, value, workspace=ws)
        lib.push_wait(flags, nflags, value, 1_000_000, missing)
        torch.cuda.synchronize()
        assert int(missing.item()) == 0
        assert (flags.cpu().numpy() == value).all()
        assert np.array_equal(to_bits(dst), to_bits(C))
        assert_bf16_launch(lib, A, W, wl, to_bits(dst), what=f"push value {value}")
