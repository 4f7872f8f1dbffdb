"""Kernel resource metadata read from the built libkq.so (tests only).

The HIP build embeds one gfx950 code object in the library's .hip_fatbin
section as a clang offload bundle.  This module extracts it with the LLVM
tools shipped with ROCm and reads each kernel's AMDGPU metadata note: its
static LDS (group segment) size and its VGPR count.  Tests use these to
check launch plans against what the compiler actually allocated.
"""
from __future__ import annotations

import functools
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quant_weight_matvec_amd", "libkq.so")
LLVM = "/opt/rocm/llvm/bin"


def _tool(name: str) -> str:
    p = os.path.join(LLVM, name)
    if os.path.exists(p):
        return p
    q = shutil.which(name)
    if not q:
        pytest.skip(f"{name} not available")
    return q


@functools.lru_cache(maxsize=1)
def kernels() -> dict[str, dict[str, int]]:
    """{mangled kernel name: {"lds": static LDS bytes, "vgpr": VGPRs, "agpr": AGPRs}}."""
    if not os.path.exists(LIB):
        pytest.skip("libkq.so is not built")
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    notes = ""
    with tempfile.TemporaryDirectory() as d:
        fb = os.path.join(d, "fb.bin")
        subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fb}", LIB,
                        os.path.join(d, "stripped")], check=True, capture_output=True)
        data = open(fb, "rb").read()
        # one bundle per source file, back to back (aligned) in the section
        starts = [m.start() for m in re.finditer(re.escape(magic), data)]
        for i, a in enumerate(starts):
            b = starts[i + 1] if i + 1 < len(starts) else len(data)
            bundle, co = os.path.join(d, f"b{i}.bin"), os.path.join(d, f"co{i}.o")
            with open(bundle, "wb") as f:
                f.write(data[a:b])
            subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o",
                            f"--input={bundle}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                            f"--output={co}"], check=True, capture_output=True)
            notes += subprocess.run([_tool("llvm-readelf"), "--notes", co], check=True,
                                    capture_output=True, text=True).stdout
    out: dict[str, dict[str, int]] = {}
    # each kernel's metadata is a YAML mapping; fields precede or follow .name
    for block in re.split(r"\n\s*-\s+\.", notes):
        name = re.search(r"\.name:\s+(\S+)", "." + block)
        if not name or ".symbol:" not in block:
            continue
        def field(key):
            m = re.search(rf"\.{key}:\s+(\d+)", "." + block)
            return int(m.group(1)) if m else 0
        out[name.group(1)] = {"lds": field("group_segment_fixed_size"),
                              "vgpr": field("vgpr_count"), "agpr": field("agpr_count")}
    assert out, "no kernel metadata found in the code object"
    return out


def max_static_lds(pattern: str) -> int:
    ks = [v["lds"] for n, v in kernels().items() if re.search(pattern, n)]
    assert ks, f"no kernel matches {pattern}"
    return max(ks)
