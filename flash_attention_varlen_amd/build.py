"""Build libmi_attn.so (HIP kernels for gfx950 + the C-ABI front end) in-tree.

    python -m flash_attention_varlen_amd.build

hipcc compiles every source for gfx950 only.  Packed fp32 VALU instructions
are switched off (``-packed-fp32-ops``); hipcc's host pass warns that it does
not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmi_attn.so")
SOURCES = [os.path.join(CSRC, "attn_fwd.hip"), os.path.join(CSRC, "mi_attn.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile the shared library; returns its path.  Always recompiles."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-pass-failed", "-Wno-unused-function",
           "-I", INCLUDE, "-I", CSRC, "-x", "hip", SOURCES[0], "-x", "hip", SOURCES[1],
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
