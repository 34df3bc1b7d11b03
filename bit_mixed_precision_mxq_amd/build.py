"""Build libmxq.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m bit_mixed_precision_mxq_amd.build   (or build_library() from Python)
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmxq.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["api.cpp", "quantize.hip", "select.hip", "attn_mixed.hip", "attn_short.hip", "decode.hip", "kvcache.hip"]
ARCH = os.environ.get("MXQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
        # packed fp32 VALU ops are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(os.path.dirname(HERE), "include"),
    ]


# per-file flags: the attention kernel never sees NaN scores (finite or -inf),
# so NaN semantics are relaxed there to drop canonicalising moves around fmaxf
# The attention kernels run with IEEE mode off (scores are never NaN).  The
# long kernel's loop is sensitive to where its branch targets fall in the
# instruction fetch blocks (up to 6% between layouts with the same code), so
# every block entered only by a jump starts on a 32-byte boundary (the padding
# sits behind unconditional branches and never runs): its speed no longer
# moves when code before the loop changes.
_ATTN = ["-fno-honor-nans", "-mno-amdgpu-ieee"]
EXTRA = {"attn_mixed.hip": _ATTN + ["-mllvm", "-align-all-nofallthru-blocks=5"], "attn_short.hip": _ATTN}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *_flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    """Compile every source and link libmxq.so next to this file.  Always
    rebuilds (the build is a few seconds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
