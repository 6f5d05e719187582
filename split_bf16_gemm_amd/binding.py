"""ctypes binding of the C ABI in include/lowm.h.

Argument marshalling only: every step of the product runs in the HIP kernels
of liblowm.so.  PyTorch supplies device memory and the current stream.  There
is no fallback: when the library is not built, or a call fails, this raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional

import torch

LIBDIR = Path(__file__).resolve().parent / "_lib"

LOWM_OK = 0
LOWM_ERR_INVALID_ARG = -1
LOWM_ERR_UNSUPPORTED = -2
LOWM_ERR_WORKSPACE = -3
LOWM_ERR_LAUNCH = -4
LOWM_ERR_SCRATCH = -5
SCRATCH_BYTES = 16 << 20
LOWM_STAGE_LDS = 0
LOWM_STAGE_REG = 1
LOWM_STAGE_LINE = 3
LOWM_STAGE_PANEL = 4
LOWM_STAGE_QUARTER = 5
LOWM_STAGE_QUARTER_ROWS = 6
MAX_M = 64
MAX_SPLIT_K = 256

# stall sites of the stress build
SITE_ENTRY = 1
SITE_STAGE_READ = 2
SITE_REDUCE = 4
SITE_PUBLISH = 8
SITE_FOLD = 16
SITE_LATE_PUBLISH = 32   # arrive first, store the partial after the stall


class Tactic(ctypes.Structure):
    _fields_ = [("stage", ctypes.c_int), ("rows", ctypes.c_int), ("waves", ctypes.c_int),
                ("unroll", ctypes.c_int), ("stages", ctypes.c_int)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}

    def __repr__(self) -> str:
        st = {LOWM_STAGE_LDS: "lds", LOWM_STAGE_REG: "reg", LOWM_STAGE_LINE: "line",
              LOWM_STAGE_PANEL: "panel", LOWM_STAGE_QUARTER: "quarter",
              LOWM_STAGE_QUARTER_ROWS: "qrows"}.get(self.stage, str(self.stage))
        return (f"Tactic({st}, rows={self.rows}, waves={self.waves}, "
                f"unroll={self.unroll}, stages={self.stages})")


def tactic(stage: str, rows: int, unroll: int, stages: int, waves: int = 4) -> Tactic:
    code = {"lds": LOWM_STAGE_LDS, "reg": LOWM_STAGE_REG, "line": LOWM_STAGE_LINE,
            "panel": LOWM_STAGE_PANEL, "quarter": LOWM_STAGE_QUARTER,
            "qrows": LOWM_STAGE_QUARTER_ROWS}[stage]
    return Tactic(code, rows, waves, unroll, stages)


MAX_BATCH = 8


class GemmDesc(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("W", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("N", ctypes.c_int)]


class LowmError(RuntimeError):
    def __init__(self, code: int, message: str, hip_error: int = 0):
        super().__init__(f"lowm error {code}: {message}"
                         + (f" (hipError {hip_error})" if hip_error else ""))
        self.code = code
        self.hip_error = hip_error


_vp = ctypes.c_void_p
_i = ctypes.c_int
_TP = ctypes.POINTER(Tactic)


class Library:
    """One loaded build of the GEMM library (default or stress)."""

    EXPORTS = ("lowm_gemm_splitk", "lowm_gemm_splitk_f32out", "lowm_gemm_splitk_workspace_bytes",
               "lowm_strerror", "lowm_last_hip_error", "lowm_pick_tactic",
               "lowm_gemm_splitk_ex", "lowm_gemm_splitk_f32out_ex")

    def __init__(self, path: Path):
        if not path.exists():
            raise RuntimeError(
                f"{path.name} is not built; run `python -m split_bf16_gemm_amd.build` "
                "(there is no CPU fallback)")
        self.path = path
        lib = ctypes.CDLL(str(path))
        for name in ("lowm_gemm_splitk", "lowm_gemm_splitk_f32out"):
            fn = getattr(lib, name)
            fn.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]
            fn.restype = _i
        for name in ("lowm_gemm_splitk_ex", "lowm_gemm_splitk_f32out_ex"):
            fn = getattr(lib, name)
            fn.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _TP]
            fn.restype = _i
        lib.lowm_gemm_splitk_workspace_bytes.argtypes = [_i, _i, _i, _i]
        lib.lowm_gemm_splitk_workspace_bytes.restype = ctypes.c_size_t
        lib.lowm_strerror.argtypes = [_i]
        lib.lowm_strerror.restype = ctypes.c_char_p
        lib.lowm_last_hip_error.argtypes = []
        lib.lowm_last_hip_error.restype = _i
        lib.lowm_pick_tactic.argtypes = [_i, _i, _i, _i, _TP]
        lib.lowm_pick_tactic.restype = _i
        lib.lowm_check_launch.argtypes = [_i, _i, _i, _i, _i, _TP]
        lib.lowm_check_launch.restype = _i
        lib.lowm_pick_split_k.argtypes = [_i, _i, _i, ctypes.POINTER(_i)]
        lib.lowm_pick_split_k.restype = _i
        lib.lowm_gemm_splitk_noalloc.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp]
        lib.lowm_gemm_splitk_noalloc.restype = _i
        lib.lowm_gemm_splitk_push.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _i, _vp,
                                              ctypes.c_uint32, _vp, ctypes.POINTER(Tactic)]
        lib.lowm_gemm_splitk_push.restype = _i
        lib.lowm_push_wait.argtypes = [_vp, _i, ctypes.c_uint32, ctypes.c_uint32, _vp, _vp]
        lib.lowm_push_wait.restype = _i
        lib.lowm_gemm_splitk_batched.argtypes = [ctypes.POINTER(GemmDesc), _i, _i, _i, _i, _vp,
                                                 _vp]
        lib.lowm_gemm_splitk_batched.restype = _i
        lib.lowm_gemm_splitk_batched_workspace_bytes.argtypes = [ctypes.POINTER(GemmDesc), _i,
                                                                 _i, _i, _i]
        lib.lowm_gemm_splitk_batched_workspace_bytes.restype = ctypes.c_size_t
        lib.lowm_workspace_status.argtypes = [_vp, _i, _vp, ctypes.POINTER(_i),
                                              ctypes.POINTER(_i)]
        lib.lowm_workspace_status.restype = _i
        self.has_stress = hasattr(lib, "lowm_stress_configure")
        if self.has_stress:
            lib.lowm_stress_configure.argtypes = [ctypes.c_uint, _i, _i, _i, _i, _i, ctypes.c_uint]
            lib.lowm_stress_configure.restype = _i
            lib.lowm_stress_trace.argtypes = [_vp, ctypes.c_size_t]
            lib.lowm_stress_trace.restype = _i
        self.lib = lib

    # -- host-only queries ------------------------------------------------
    def strerror(self, code: int) -> str:
        return self.lib.lowm_strerror(code).decode()

    def workspace_bytes(self, M: int, N: int, K: int, split_k: int) -> int:
        return int(self.lib.lowm_gemm_splitk_workspace_bytes(M, N, K, split_k))

    def pick_tactic(self, M: int, N: int, K: int, split_k: int) -> Tactic:
        t = Tactic()
        self.check(self.lib.lowm_pick_tactic(M, N, K, split_k, ctypes.byref(t)))
        return t

    def pick_split_k(self, M: int, N: int, K: int) -> int:
        """Host-only: the split_k measured fastest for these sizes."""
        s = _i(0)
        self.check(self.lib.lowm_pick_split_k(M, N, K, ctypes.byref(s)))
        return s.value

    def check_launch(self, M: int, N: int, K: int, split_k: int, f32out: bool = False,
                     tactic: Optional[Tactic] = None) -> int:
        """Host-only: the code a launch would return before running (0 = runs)."""
        return self.lib.lowm_check_launch(M, N, K, split_k, int(f32out),
                                          None if tactic is None else ctypes.byref(tactic))

    def check(self, rc: int):
        if rc != LOWM_OK:
            hip = self.lib.lowm_last_hip_error() if rc == LOWM_ERR_LAUNCH else 0
            raise LowmError(rc, self.strerror(rc), hip)

    # -- raw calls (pointers as ints) ------------------------------------
    def call_raw(self, A: int, W: int, C: int, M: int, N: int, K: int, split_k: int,
                 workspace: int, stream: int, f32out: bool = False,
                 tactic: Optional[Tactic] = None) -> int:
        if tactic is None:
            fn = self.lib.lowm_gemm_splitk_f32out if f32out else self.lib.lowm_gemm_splitk
            return fn(A, W, C, M, N, K, split_k, workspace, stream)
        fn = self.lib.lowm_gemm_splitk_f32out_ex if f32out else self.lib.lowm_gemm_splitk_ex
        return fn(A, W, C, M, N, K, split_k, workspace, stream, ctypes.byref(tactic))

    # -- torch-facing call -------------------------------------------------
    def gemm(self, A: torch.Tensor, W: torch.Tensor, split_k: int = 1,
             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             out_dtype: torch.dtype = torch.bfloat16, tactic: Optional[Tactic] = None,
             stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """C = A @ W.T on the GPU (A [M,K], W [N,K] bf16) through the C ABI."""
        M, N, K = self._operands(A, W)
        f32out = out_dtype == torch.float32
        out = self._out(out, M, N, out_dtype, A.device)
        ws_ptr = self._workspace_ptr(workspace, M, N, K, split_k)
        s = stream if stream is not None else torch.cuda.current_stream(A.device)
        rc = self.call_raw(A.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K, split_k,
                           ws_ptr, s.cuda_stream, f32out, tactic)
        self.check(rc)
        return out

    def gemm_noalloc(self, A: torch.Tensor, W: torch.Tensor, split_k: int = 1,
                     out: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """C = A @ W.T (bf16) through lowm_gemm_splitk_noalloc: the split-K
        workspace is the library's built-in scratch, so the C call allocates
        nothing (pass `out` to keep this call allocation-free as well)."""
        M, N, K = self._operands(A, W)
        out = self._out(out, M, N, torch.bfloat16, A.device)
        s = stream if stream is not None else torch.cuda.current_stream(A.device)
        self.check(self.lib.lowm_gemm_splitk_noalloc(A.data_ptr(), W.data_ptr(), out.data_ptr(),
                                                     M, N, K, split_k, s.cuda_stream))
        return out

    @staticmethod
    def _operands(A, W):
        if A.dim() != 2 or W.dim() != 2 or A.shape[1] != W.shape[1]:
            raise ValueError(f"shapes {tuple(A.shape)} and {tuple(W.shape)} do not chain")
        if A.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
            raise TypeError("A and W must be bfloat16")
        if not (A.is_cuda and W.is_cuda):
            raise ValueError("A and W must be on the GPU")
        if not (A.is_contiguous() and W.is_contiguous()):
            raise ValueError("A and W must be contiguous row-major")
        return A.shape[0], W.shape[0], A.shape[1]

    @staticmethod
    def _out(out, M, N, dtype, device):
        if out is None:
            out = torch.empty((M, N), dtype=dtype, device=device)
        if out.shape != (M, N) or out.dtype != dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous [M, N] tensor of out_dtype")
        return out

    def _workspace_ptr(self, workspace, M, N, K, split_k) -> int:
        if split_k <= 1:
            return 0
        need = self.workspace_bytes(M, N, K, split_k)
        if need == 0:   # sizes the launch rejects: report its error code
            self.check(self.check_launch(M, N, K, split_k))
        if workspace is None:
            raise ValueError(f"split_k={split_k} needs a zeroed workspace of {need} bytes "
                             "(make_workspace)")
        if workspace.numel() * workspace.element_size() < need or not workspace.is_cuda:
            raise ValueError(f"workspace smaller than {need} bytes")
        return workspace.data_ptr()

    def gemm_push(self, A, W, split_k, push, flags, flag_value, out=None, workspace=None,
                  tactic=None, stream=None):
        """C = A @ W.T with the push epilogue: every output tile also goes to
        `push` (a bf16 [M, >= N] view whose rows may be strided, last dim
        contiguous) and then flag j (columns 16j..16j+15) of `flags` (int32
        or uint32 bits) is set to flag_value."""
        M, N, K = self._operands(A, W)
        out = self._out(out, M, N, torch.bfloat16, A.device)
        if push.dtype != torch.bfloat16 or push.dim() != 2 or push.shape[0] != M or \
                push.shape[1] < N or push.stride(1) != 1 or not push.is_cuda:
            raise ValueError("push must be a bf16 GPU view of shape [M, >= N], unit column stride")
        if flags.dtype != torch.int32 or flags.numel() < (N + 15) // 16 or not flags.is_cuda \
                or not flags.is_contiguous():
            raise ValueError(f"flags must be a contiguous int32 GPU tensor of >= {(N + 15) // 16}")
        ws_ptr = self._workspace_ptr(workspace, M, N, K, split_k)
        s = stream if stream is not None else torch.cuda.current_stream(A.device)
        tp = ctypes.byref(tactic) if tactic is not None else None
        self.check(self.lib.lowm_gemm_splitk_push(
            A.data_ptr(), W.data_ptr(), out.data_ptr(), M, N, K, split_k, ws_ptr,
            push.data_ptr(), push.stride(0), flags.data_ptr(), flag_value, s.cuda_stream, tp))
        return out

    def push_wait(self, flags, n_flags: int, flag_value: int, timeout_us: int, missing,
                  stream=None):
        """Enqueue the bounded wait for flags[0:n_flags] == flag_value; the count
        of flags not seen set lands in missing[0] (an int32 GPU tensor)."""
        if missing.dtype != torch.int32 or not missing.is_cuda or flags.dtype != torch.int32:
            raise ValueError("flags and missing must be int32 GPU tensors")
        if not flags.is_cuda or not flags.is_contiguous() or not 1 <= n_flags <= flags.numel():
            raise ValueError(f"flags must be a contiguous GPU tensor of at least n_flags = "
                             f"{n_flags} (>= 1) words")
        s = stream if stream is not None else torch.cuda.current_stream(flags.device)
        self.check(self.lib.lowm_push_wait(flags.data_ptr(), n_flags, flag_value, timeout_us,
                                           missing.data_ptr(), s.cuda_stream))

    @staticmethod
    def descs(As, Ws, Cs):
        """A ctypes array of lowm_gemm_desc for lists of GPU tensors."""
        arr = (GemmDesc * len(Ws))()
        for g, (A, W, C) in enumerate(zip(As, Ws, Cs)):
            arr[g] = GemmDesc(A.data_ptr(), W.data_ptr(), C.data_ptr(), W.shape[0])
        return arr

    def batched_workspace_bytes(self, M: int, Ns, K: int, split_k: int) -> int:
        """Bytes of a batch's workspace: the single-GEMM workspaces of its
        GEMMs, back to back in batch order (0 for split_k 1 or a bad batch)."""
        arr = (GemmDesc * max(1, len(Ns)))()
        for g, N in enumerate(Ns):
            arr[g] = GemmDesc(None, None, None, N)
        return int(self.lib.lowm_gemm_splitk_batched_workspace_bytes(arr, len(Ns), M, K, split_k))

    def gemm_batched(self, As, Ws, split_k: int = 1, outs=None, workspace=None, stream=None):
        """[A_g @ W_g.T for each g] in one launch (bf16 out).  All A_g share M and
        K; the W_g share K; up to MAX_BATCH GEMMs."""
        if len(As) != len(Ws) or not As:
            raise ValueError("need as many A as W, at least one")
        M, K = As[0].shape
        for A, W in zip(As, Ws):
            if A.shape != (M, K) or W.dim() != 2 or W.shape[1] != K:
                raise ValueError("every A must be [M, K] and every W [N, K]")
            if A.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
                raise TypeError("A and W must be bfloat16")
            if not (A.is_cuda and W.is_cuda and A.is_contiguous() and W.is_contiguous()):
                raise ValueError("A and W must be contiguous GPU tensors")
        if outs is None:
            outs = [torch.empty((M, W.shape[0]), dtype=torch.bfloat16, device=A.device)
                    for A, W in zip(As, Ws)]
        ws_ptr = 0
        if split_k > 1:
            need = self.batched_workspace_bytes(M, [W.shape[0] for W in Ws], K, split_k)
            if workspace is None or workspace.numel() * workspace.element_size() < need:
                raise ValueError(f"split_k={split_k} needs a zeroed workspace of {need} bytes")
            ws_ptr = workspace.data_ptr()
        s = stream if stream is not None else torch.cuda.current_stream(As[0].device)
        arr = self.descs(As, Ws, outs)
        self.check(self.lib.lowm_gemm_splitk_batched(arr, len(Ws), M, K, split_k, ws_ptr,
                                                     s.cuda_stream))
        return outs

    def make_workspace(self, M: int, N: int, K: int, split_k: int,
                       device="cuda") -> Optional[torch.Tensor]:
        """A zeroed workspace for these sizes (None when split_k == 1)."""
        n = self.workspace_bytes(M, N, K, split_k)
        if n == 0:
            return None
        return torch.zeros(n, dtype=torch.uint8, device=device)

    def workspace_status(self, workspace: torch.Tensor, N: int, stream=None) -> tuple:
        """(faulted tiles, tiles with a non-zero arrival count) of a workspace
        last used by a launch with N output columns, once ``stream`` (default:
        the current one) has drained."""
        if workspace is None or not workspace.is_cuda:
            raise ValueError("workspace_status needs the device workspace tensor")
        if workspace.numel() * workspace.element_size() < 256 * ((N + 15) // 16):
            raise ValueError(f"the workspace is too small for N={N}")
        s = stream if stream is not None else torch.cuda.current_stream(workspace.device)
        faulted, open_ = ctypes.c_int(0), ctypes.c_int(0)
        with torch.cuda.device(workspace.device):
            self.check(self.lib.lowm_workspace_status(workspace.data_ptr(), N, s.cuda_stream,
                                                      ctypes.byref(faulted), ctypes.byref(open_)))
        return faulted.value, open_.value

    TRACE_SLOTS = 10    # entry, first stage, loop end, reduced, arrived, end, CU, XCD, tile, rank

    def trace(self, buf: Optional[torch.Tensor]):
        """Stress build: per-workgroup timestamps into ``buf`` (int64 device
        tensor, TRACE_SLOTS per workgroup), or stop tracing with None.  A
        launch with more workgroups than ``buf`` holds is refused."""
        if not self.has_stress:
            raise RuntimeError(f"{self.path.name} is not a stress build")
        if buf is None:
            self.check(self.lib.lowm_stress_trace(None, 0))
            return
        if buf.dtype != torch.int64 or not buf.is_cuda or not buf.is_contiguous():
            raise ValueError("the trace buffer must be a contiguous int64 GPU tensor")
        self.check(self.lib.lowm_stress_trace(buf.data_ptr(), buf.numel() // self.TRACE_SLOTS))

    def configure_stress(self, sites: int = 0, rank: int = -1, wave: int = -1,
                         tile_mod: int = 0, tile_sel: int = 0, step: int = -1,
                         delay_ns: int = 0):
        if not self.has_stress:
            raise RuntimeError(f"{self.path.name} is not a stress build")
        self.check(self.lib.lowm_stress_configure(sites, rank, wave, tile_mod, tile_sel, step,
                                                  delay_ns))


_libs: dict = {}


def load(kind: str = "default") -> Library:
    """The built library: kind 'default' (liblowm.so), 'stress' or 'fenced'."""
    if kind not in _libs:
        name = {"default": "liblowm.so", "stress": "liblowm_stress.so",
                "fenced": "liblowm_fenced.so"}[kind]
        _libs[kind] = Library(LIBDIR / name)
    return _libs[kind]


def gemm(A, W, split_k=1, **kw):
    return load().gemm(A, W, split_k, **kw)


def workspace_bytes(M, N, K, split_k):
    return load().workspace_bytes(M, N, K, split_k)


def gemm_batched(As, Ws, split_k=1, **kw):
    return load().gemm_batched(As, Ws, split_k, **kw)


def batched_workspace_bytes(M, Ns, K, split_k):
    return load().batched_workspace_bytes(M, Ns, K, split_k)


def pick_split_k(M, N, K):
    return load().pick_split_k(M, N, K)


def make_workspace(M, N, K, split_k, device="cuda"):
    return load().make_workspace(M, N, K, split_k, device)


def counter_bytes(N: int) -> int:
    """Bytes of the counter region at the start of a workspace: one counter
    per 16 columns of C, each on its own 256-byte line (lowm.h)."""
    return 256 * ((N + 15) // 16)


class BwProbe:
    """Streaming read / copy kernels (libbwprobe.so) for the HBM ceiling."""

    def __init__(self):
        path = LIBDIR / "libbwprobe.so"
        if not path.exists():
            raise RuntimeError("libbwprobe.so is not built")
        lib = ctypes.CDLL(str(path))
        lib.bwprobe_read.argtypes = [_vp, ctypes.c_size_t, _vp, _i, _vp]
        lib.bwprobe_read.restype = _i
        lib.bwprobe_copy.argtypes = [_vp, _vp, ctypes.c_size_t, _i, _vp]
        lib.bwprobe_copy.restype = _i
        lib.bwprobe_empty.argtypes = [_i, _vp]
        lib.bwprobe_empty.restype = _i
        self.lib = lib

    def empty(self, blocks: int):
        rc = self.lib.bwprobe_empty(blocks, torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"bwprobe_empty failed: hipError {rc}")

    def read(self, src: torch.Tensor, sink: torch.Tensor, blocks: int):
        n = src.numel() * src.element_size()
        rc = self.lib.bwprobe_read(src.data_ptr(), n, sink.data_ptr(), blocks,
                                   torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"bwprobe_read failed: hipError {rc}")

    def copy(self, src: torch.Tensor, dst: torch.Tensor, blocks: int):
        n = src.numel() * src.element_size()
        rc = self.lib.bwprobe_copy(src.data_ptr(), dst.data_ptr(), n, blocks,
                                   torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"bwprobe_copy failed: hipError {rc}")
