"""Every kernel in the built library (and in its schedule variants) uses no
scratch memory: no private segment and no vector registers spilled to it, so
no kernel pays for spill traffic.  (Scalar registers that the compiler parks
in lanes of a vector register are not scratch and are allowed.)  Read from
the library's own device code objects (built here), through their AMDGPU
metadata notes."""
import os
import re
import struct
import subprocess

import pytest

import flash_attention_varlen_amd as fav
from flash_attention_varlen_amd import build as fav_build

READELF = "/opt/rocm/llvm/bin/llvm-readelf"
OBJCOPY = "/opt/rocm/llvm/bin/llvm-objcopy"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _code_objects(lib_path, tmp_path):
    """The gfx950 code objects in the library's .hip_fatbin section (one
    clang offload bundle per translation unit)."""
    fat = tmp_path / "fatbin.bin"
    r = subprocess.run([OBJCOPY, "--dump-section", f".hip_fatbin={fat}", lib_path,
                        str(tmp_path / "stripped.so")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    data = fat.read_bytes()
    objs, pos = [], 0
    while True:
        i = data.find(BUNDLE_MAGIC, pos)
        if i < 0:
            break
        n = struct.unpack_from("<Q", data, i + len(BUNDLE_MAGIC))[0]
        p = i + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tl].decode()
            p += tl
            if triple.endswith("gfx950"):
                objs.append(data[i + off:i + off + size])
        pos = i + 1
    return objs


def _kernel_resources(obj, path):
    path.write_bytes(obj)
    r = subprocess.run([READELF, "--notes", str(path)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = r.stdout
    names = re.findall(r"^\s+\.name:\s+(\S+)", text, re.M)
    fields = {k: [int(x) for x in re.findall(rf"^\s+\.{k}:\s+(\d+)", text, re.M)]
              for k in ("private_segment_fixed_size", "vgpr_spill_count", "sgpr_spill_count")}
    for k, v in fields.items():
        assert len(v) == len(names), (k, len(v), len(names))
    return [(names[i], {k: v[i] for k, v in fields.items()}) for i in range(len(names))]


def _libraries():
    libs = [fav.LIB_PATH]
    libs += [fav_build.variant_path(n) for n in sorted(fav_build.VARIANTS)]
    return libs


@pytest.mark.skipif(not (os.path.exists(READELF) and os.path.exists(OBJCOPY)),
                    reason="needs the ROCm LLVM tools")
@pytest.mark.parametrize("lib", _libraries(), ids=lambda p: os.path.basename(p))
def test_no_kernel_uses_scratch(lib, tmp_path):
    if not os.path.exists(lib):
        pytest.skip(f"{lib} is not built")
    objs = _code_objects(lib, tmp_path)
    assert objs, "no gfx950 code object in the library"
    kernels = []
    for i, obj in enumerate(objs):
        kernels += _kernel_resources(obj, tmp_path / f"co{i}.o")
    assert len(kernels) > 20
    bad = [(n, r) for n, r in kernels if r["private_segment_fixed_size"] or r["vgpr_spill_count"]]
    assert not bad, f"{len(bad)} kernel(s) use scratch: {bad[:4]}"
