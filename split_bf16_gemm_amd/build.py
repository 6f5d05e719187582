"""Compile the HIP libraries of the package for gfx950, in-tree.

    python -m split_bf16_gemm_amd.build

produces, under split_bf16_gemm_amd/_lib/:
  liblowm.so         the GEMM (C ABI of include/lowm.h)
  liblowm_stress.so  the same sources with -DLOWM_STRESS (stall injection)
  libbwprobe.so      streaming read/copy kernels for the HBM ceiling

and, only when named (python -m split_bf16_gemm_amd.build liblowm_fenced.so):
  liblowm_fenced.so  the same sources with -DLOWM_FENCED (a release arrival
                     and an acquire fence in the owner; a comparison build)

Each library is linked from objects compiled separately (the kernels of each
output kind are a translation unit of their own), all in parallel.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIBDIR = PKG / "_lib"
OBJDIR = LIBDIR / "obj"
INCLUDE = ROOT / "include"

ARCH = "gfx950"
# Packed-fp32 instructions are disabled for every HIP object built here.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-pass-failed", f"-I{INCLUDE}"]

GEMM_SOURCES = ["lowm_host.hip", "lowm_inst_bf16.hip", "lowm_inst_f32.hip",
                "lowm_inst_push.hip"]
TARGETS = {
    "liblowm.so": (GEMM_SOURCES, []),
    "liblowm_stress.so": (GEMM_SOURCES, ["-DLOWM_STRESS"]),
    "libbwprobe.so": (["bwprobe.hip"], []),
}
# built only when named
OPTIONAL = {
    "liblowm_fenced.so": (GEMM_SOURCES, ["-DLOWM_FENCED"]),
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(path).exists():
        raise RuntimeError("hipcc not found (ROCm is required to build)")
    return path


def _run(cmd: list[str], what: str, verbose: bool):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that note.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    log = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{' '.join(cmd)}\n{log}")
    if verbose and log.strip():
        print(log, file=sys.stderr)


def _object(lib: str, src: str) -> Path:
    return OBJDIR / f"{Path(lib).stem}.{Path(src).stem}.o"


def _compile(lib: str, src: str, extra: list[str], verbose: bool) -> Path:
    out = _object(lib, src)
    tmp = out.with_suffix(f".tmp{os.getpid()}.o")
    _run([hipcc(), *COMMON, *extra, "-c", "-o", str(tmp), str(CSRC / src)],
         f"compiling {src} for {lib}", verbose)
    os.replace(tmp, out)
    return out


def _link(lib: str, verbose: bool) -> Path:
    sources, _ = {**TARGETS, **OPTIONAL}[lib]
    out = LIBDIR / lib
    tmp = LIBDIR / f"{lib}.tmp{os.getpid()}"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
          *[str(_object(lib, s)) for s in sources]], f"linking {lib}", verbose)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, only: list[str] | None = None) -> list[Path]:
    """Compile every library (objects in parallel) and return their paths."""
    LIBDIR.mkdir(exist_ok=True)
    OBJDIR.mkdir(exist_ok=True)
    every = {**TARGETS, **OPTIONAL}
    unknown = [l for l in (only or []) if l not in every]
    if unknown:
        raise ValueError(f"unknown libraries {unknown}; known: {sorted(every)}")
    libs = [l for l in TARGETS if only is None or l in only] + \
        [l for l in OPTIONAL if only is not None and l in only]
    jobs = [(lib, src, every[lib][1]) for lib in libs for src in every[lib][0]]
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda j: _compile(*j, verbose), jobs))
    return [_link(lib, verbose) for lib in libs]


if __name__ == "__main__":
    names = [a for a in sys.argv[1:] if not a.startswith("-")]
    for p in build(verbose=True, only=names or None):
        print(p)
