"""Compile the HIP libraries of the package for gfx950, in-tree.

    python -m split_bf16_gemm_amd.build

produces, under split_bf16_gemm_amd/_lib/:
  liblowm.so         the GEMM (C ABI of include/lowm.h)
  liblowm_stress.so  the same source with -DLOWM_STRESS (stall injection)
  libbwprobe.so      streaming read/copy kernels for the HBM ceiling
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
INCLUDE = ROOT / "include"

ARCH = "gfx950"
# Packed-fp32 instructions are disabled for every HIP object built here.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", f"-I{INCLUDE}"]

TARGETS = {
    "liblowm.so": (["lowm_splitk.hip"], []),
    "liblowm_stress.so": (["lowm_splitk.hip"], ["-DLOWM_STRESS"]),
    "libbwprobe.so": (["bwprobe.hip"], []),
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(path).exists():
        raise RuntimeError("hipcc not found (ROCm is required to build)")
    return path


def _build_one(name: str, verbose: bool) -> Path:
    sources, extra = TARGETS[name]
    out = LIBDIR / name
    tmp = LIBDIR / f"{name}.tmp{os.getpid()}"
    cmd = [hipcc(), *COMMON, *extra, "-o", str(tmp), *[str(CSRC / s) for s in sources]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that note.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    log = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"building {name} failed:\n{' '.join(cmd)}\n{log}")
    if verbose and log.strip():
        print(log, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> list[Path]:
    """Compile every library (in parallel) and return their paths."""
    LIBDIR.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(TARGETS)) as ex:
        return list(ex.map(lambda n: _build_one(n, verbose), TARGETS))


if __name__ == "__main__":
    for p in build(verbose=True):
        print(p)
