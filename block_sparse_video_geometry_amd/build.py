"""Build libvsa.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python block_sparse_video_geometry_amd/build.py [--jobs N]

(run by path: importing the package loads the library this script builds)

Objects go to _build/ at the repository root; the library to
block_sparse_video_geometry_amd/_lib/libvsa.so.  Always recompiles.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIBDIR = PKG / "_lib"
LIB = LIBDIR / "libvsa.so"
BUILD = ROOT / "_build"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", str(ROOT / "include"), "-I", str(CSRC),
    "-Wall", "-Wno-unused-function",
    # packed fp32 ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
SOURCES = ["vsa_plan.cpp", "vsa_forward.hip", "k_pool.hip", "k_coarse.hip", "k_select.hip", "k_extra.hip",
           "k_fine.hip", "k_reblock.hip"]
# Per-file extras.  The fine kernel never sees a NaN (finite inputs; masked logits are -inf),
# so fmaxf needs no quieting of signalling NaNs.
EXTRA = {"k_fine.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> Path:
    obj = BUILD / (src + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-c", str(CSRC / src), "-o", str(obj)]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "c++"] + [c for c in COMMON if not c.startswith("--offload")] + \
              ["-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    LIBDIR.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", str(tmp)] + \
          [str(o) for o in objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args()
    try:
        build(a.jobs, verbose=True)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
