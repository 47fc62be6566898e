"""Build the HIP library libfg.so for gfx950 (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIB_DIR, "libfg.so")
SOURCES = [os.path.join(CSRC, "fg.hip")]
HEADERS = [os.path.join(CSRC, n) for n in ("fg_sync.hpp", "fg_gemm.hpp", "fg_plan.hpp", "fg_kernels.hpp", "fg_combine.hpp")] + [
    os.path.join(ROOT, "include", "fg.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept out of every code object on this part
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libfg.so; always recompiles."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libfg.so")
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_path: str) -> str:
    """Write the gfx950 assembly of the library (for inspection of the kernels)."""
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-S",
           *SOURCES, "-o", out_path]
    subprocess.run(cmd, check=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
