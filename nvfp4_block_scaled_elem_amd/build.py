"""Build libnvfp4.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

Flags: -O3 for gfx950 only; -ffp-contract=off so that every floating-point expression is the IEEE
operation it spells (fused multiply-adds only where fma() is written); packed-FP32 instructions off;
symbols hidden except the C ABI.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4.so")
SOURCES = ["quant_kernels.hip", "soar_kernel.hip", "gemm_kernels.hip", "gptq_kernels.hip", "api.cpp", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
    "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-I" + os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile the library to `out`; `defines` are extra -D settings of the tuning knobs in launch.hpp."""
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    r = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
