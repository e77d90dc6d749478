"""Compile the HIP sources of this package for gfx950.

Every ``csrc/*.hip`` file and ``csrc/abi.cpp`` is compiled by hipcc in
parallel, then linked into ``librope_mi355x.so`` next to this file (the
library of include/rope_mi355x.h).  ``calib/calib.hip`` becomes
``librope_calib.so`` (include/rope_calib.h): measurement kernels the
benchmark times beside the library's, not part of it.  Packed fp32
instructions are disabled for all device code.
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
INCLUDE = ROOT / "include"
LIBRARY = PKG / "librope_mi355x.so"
CALIB_SOURCE = PKG / "calib" / "calib.hip"
CALIB_LIBRARY = PKG / "librope_calib.so"
BUILD_DIR = PKG / "_build"

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(exe).exists():
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build")
    return exe


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip")) + [CSRC / "abi.cpp"]


# Per-file extra flags.  The fused attention kernels never produce or test a
# NaN (masked scores are -inf, which stays honoured); without
# -fno-honor-nans every fmaxf on a matrix-core result gets a NaN-quieting
# v_max_f32 x, x, x in front of it.  Host-side argument validation (abi.cpp)
# does test for NaN and keeps IEEE semantics.
FILE_FLAGS = {name: ["-fno-honor-nans"] for name in ("flash_fwd_bf16.hip", "flash_fwd_pp.hip")}


def _compile(src: Path) -> Path:
    obj = BUILD_DIR / (src.name + ".o")
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(src.name, []), "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs: list[Path], library: Path) -> Path:
    tmp = library.with_name(library.name + f".tmp{os.getpid()}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, library)
    return library


def build(jobs: int | None = None) -> Path:
    """Compile and link both libraries; returns the path of the RoPE
    library.  Always rebuilds."""
    BUILD_DIR.mkdir(exist_ok=True)
    srcs = sources() + [CALIB_SOURCE]
    with ThreadPoolExecutor(max_workers=jobs or min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIBRARY)
    _link(objs[-1:], CALIB_LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build())
