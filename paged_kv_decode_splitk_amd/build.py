"""Build the HIP library ``libpkd.so`` in-tree with hipcc for gfx950.

``python -m paged_kv_decode_splitk_amd.build`` compiles every ``csrc/*.hip``
into one shared object next to this file. The flags keep IEEE float32
division and denormals (the FP8 / NVFP4 encoders are bit-exact), switch off
packed-FP32 instruction selection, and hide every symbol except the C ABI.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libpkd.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = os.environ.get("PKD_OFFLOAD_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def hipcc_command(out=LIB_PATH):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [
        hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in VGPRs: the accumulators are also scaled by VALU code,
        # and AGPR-resident ones are copied to VGPRs and back around it
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", os.path.join(ROOT, "include"),
        *os.environ.get("PKD_EXTRA_HIPCC_FLAGS", "").split(),
        "-o", out, *sources(),
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always, even when a built copy exists)."""
    tmp = LIB_PATH + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and res.stderr.strip():
        # the host pass does not know the packed-fp32 feature; that warning is harmless
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            print("\n".join(lines))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


STANDALONE_SRC = os.path.join(ROOT, "tests", "standalone", "decode_tiny.cpp")
STANDALONE_BIN = os.path.join(ROOT, "tests", "standalone", "decode_tiny")


def build_standalone(verbose: bool = False) -> str:
    """Compile the standalone C++ test of the C ABI (host code only), linked
    against the in-tree library with an rpath to it."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"),
           STANDALONE_SRC, "-L", HERE, "-lpkd",
           "-Wl,-rpath,$ORIGIN/../../paged_kv_decode_splitk_amd", "-o", STANDALONE_BIN]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc (standalone test) failed with status {res.returncode}")
    return STANDALONE_BIN


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_standalone(verbose=True))
