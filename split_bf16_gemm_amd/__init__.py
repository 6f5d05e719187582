"""Low-M split-K bf16 GEMM for AMD Instinct MI355X (gfx950).

C = A @ W.T with A [M, K] and W [N, K] bf16, fp32 accumulation, a bf16 (or
fp32) result, K cut into split_k slices whose partials the last-arriving
slice adds in slice order.  The work runs in the HIP kernels of
``_lib/liblowm.so`` (C ABI in ``include/lowm.h``); this package only loads and
calls them.
"""
from .binding import (MAX_BATCH, BwProbe, GemmDesc, Library, LowmError, Tactic,
                      batched_workspace_bytes, counter_bytes, gemm, gemm_batched, load,
                      make_workspace, pick_split_k, tactic, workspace_bytes)

__all__ = ["MAX_BATCH", "BwProbe", "GemmDesc", "Library", "LowmError", "Tactic",
           "batched_workspace_bytes", "counter_bytes", "gemm", "gemm_batched", "load",
           "make_workspace", "pick_split_k", "tactic", "workspace_bytes"]
