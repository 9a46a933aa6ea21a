"""Build libmoe_mi355x.so for gfx950 from csrc/*.hip with hipcc.

    python sparse_moe_transformer_way_amd/build.py

(run as a file: importing the package loads the library, which is what this
script builds).  Only the standard library is used.

Objects go to sparse_moe_transformer_way_amd/_build/, the shared library next
to this file.  Every call recompiles everything (a few seconds per file).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# -disable-promote-alloca-to-lds: private arrays never silently take LDS (the
# tiled kernels budget all of it themselves).
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build")
    return path


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    # -z defs: an unresolved symbol fails the link instead of the first load
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
