"""Build libspear_ec.so (HIP, gfx950) in place, next to this file.

    python -m quantization_error_compensation_amd.build

Each kernel file is compiled on its own (in parallel) and linked into one
shared library.  Packed fp32 VALU instructions are disabled for the device
code; the host pass warns that it does not know the feature, which is
harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libspear_ec.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "static_scratch.hip", "k_quant.hip", "k_proj.hip", "k_decode.hip",
           "k_prefill.hip", "scheduler.cpp"]
ARCH = os.environ.get("SPEAR_EC_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-file flags.  The prefill GEMM folds its matrix-core accumulators with
# vector instructions every K block; keeping the accumulators in ordinary
# VGPRs (instead of the compiler's default AGPR placement) removes a copy of
# every accumulator in and out of the AGPR file per block.
FILE_FLAGS = {"k_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every kernel source and link libspear_ec.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
