"""Build tests/hip/libmxq_testkernels.so (test-only kernels, gfx950) in-tree.

The flags match those of the attention kernel's source, so the P conversion
compiles to the same instruction sequence there and here."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "libmxq_testkernels.so")


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    arch = os.environ.get("MXQ_OFFLOAD_ARCH", "gfx950")
    tmp = OUT + ".tmp"
    cmd = [hipcc, f"--offload-arch={arch}", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans", "-mno-amdgpu-ieee",
           os.path.join(HERE, "test_kernels.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"test kernel build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
