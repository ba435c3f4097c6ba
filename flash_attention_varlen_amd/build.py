"""Build libmi_attn.so (HIP kernels for gfx950 + the C-ABI front end) in-tree.

    python -m flash_attention_varlen_amd.build

hipcc compiles every source for gfx950 only, one object per kernel instance
unit (in parallel), then links them into one shared library.  Packed fp32
VALU instructions are switched off (``-packed-fp32-ops``); hipcc's host pass
warns that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmi_attn.so")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wall", "-Wno-pass-failed", "-Wno-unused-function",
         "-Wno-cuda-compat", "-I", INCLUDE, "-I", CSRC]
# Sources compiled once each.
PLAIN = ["attn_bwd.hip", "attn_decode.hip", "bias_ranges.hip", "padding.hip", "mi_attn.cpp"]
# The forward (dispatcher + instances) is also built in schedule variants
# that only the LDS race test loads: all 16-bit kernels with two K/V slots;
# every step waiting for its own copies behind a barrier before any read;
# the four-slot kernels with copies one step less ahead.  All must give
# results bitwise equal to the shipping library.
VARIANTS = {"slots2": ["-DMI_ATTN_MAX_SLOTS=2"], "synccopies": ["-DMI_ATTN_SYNC_COPIES=1"],
            "shallow": ["-DMI_ATTN_DEEP_COPIES=0"]}
VARIANT_DIR = os.path.join(PKG, "variants")


def variant_path(name: str) -> str:
    return os.path.join(VARIANT_DIR, f"libmi_attn_{name}.so")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _instance_list(header: str, macro: str, pattern: str):
    text = open(os.path.join(CSRC, header)).read()
    body = text[text.index(f"#define {macro}(X)"):]
    body = body[:body.index("\n#define", 1)]
    return re.findall(pattern, body)


def instances():
    """(tag, type, dqk, dv) of every forward kernel instance, read from the
    MI_ATTN_FWD_INSTANCES list in attn_fwd.h."""
    return _instance_list("attn_fwd.h", "MI_ATTN_FWD_INSTANCES", r"X\((\w+), (\w+), (\d+), (\d+)\)")


def bwd_instances():
    """(tag, type, d) of every backward instance (MI_ATTN_BWD_INSTANCES in attn_bwd.h)."""
    return _instance_list("attn_bwd.h", "MI_ATTN_BWD_INSTANCES", r"X\((\w+), (\w+), (\d+)\)")


def forward_jobs(objdir: str, tag_suffix: str = "", defines=()):
    jobs = []
    obj = os.path.join(objdir, f"attn_fwd{tag_suffix}.o")
    jobs.append(([hipcc(), f"--offload-arch={ARCH}", *FLAGS, *defines, "-c", "-x", "hip",
                  os.path.join(CSRC, "attn_fwd.hip"), "-o", obj], obj))
    for tag, t, dqk, dv in instances():
        obj = os.path.join(objdir, f"attn_fwd_inst_{tag}_{dqk}_{dv}{tag_suffix}.o")
        jobs.append(([hipcc(), f"--offload-arch={ARCH}", *FLAGS, *defines,
                      f"-DMI_ATTN_INST_TAG={tag}", f"-DMI_ATTN_INST_T={t}",
                      f"-DMI_ATTN_INST_DQK={dqk}", f"-DMI_ATTN_INST_DV={dv}", "-c", "-x", "hip",
                      os.path.join(CSRC, "attn_fwd_inst.hip"), "-o", obj], obj))
    return jobs


def compile_jobs(objdir: str):
    jobs = []
    for src in PLAIN:
        obj = os.path.join(objdir, src + ".o")
        jobs.append(([hipcc(), f"--offload-arch={ARCH}", *FLAGS, "-c", "-x", "hip",
                      os.path.join(CSRC, src), "-o", obj], obj))
    for tag, t, d in bwd_instances():
        obj = os.path.join(objdir, f"attn_bwd_inst_{tag}_{d}.o")
        jobs.append(([hipcc(), f"--offload-arch={ARCH}", *FLAGS, f"-DMI_ATTN_INST_TAG={tag}",
                      f"-DMI_ATTN_INST_T={t}", f"-DMI_ATTN_INST_D={d}", "-c", "-x", "hip",
                      os.path.join(CSRC, "attn_bwd_inst.hip"), "-o", obj], obj))
    return jobs


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return r.returncode, [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]


def _link(objs, out):
    tmp = out + ".tmp"
    rc, lines = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(lines))
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int = 0, variants: bool = True) -> str:
    """Compile the shared library (and, with ``variants``, the schedule
    variants of the forward); returns the library's path.  Always recompiles."""
    jobs = jobs or min(16, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="mi_attn_build_") as objdir:
        shared = compile_jobs(objdir)
        fwd = forward_jobs(objdir)
        var = {name: forward_jobs(objdir, "_" + name, defs) for name, defs in VARIANTS.items()} \
            if variants else {}
        todo = shared + fwd + [j for js in var.values() for j in js]
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda j: _run(j[0]), todo))
        for (cmd, _), (rc, lines) in zip(todo, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
            if verbose and lines:
                print("\n".join(lines))
        _link([obj for _, obj in shared + fwd], LIB)
        if var:
            os.makedirs(VARIANT_DIR, exist_ok=True)
        for name, js in var.items():
            _link([obj for _, obj in shared + js], variant_path(name))
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
