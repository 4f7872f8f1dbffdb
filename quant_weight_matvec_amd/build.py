"""Build libkq.so (the HIP library) in-tree with hipcc for gfx950.

``build()`` compiles every source under ``csrc/`` into
``quant_weight_matvec_amd/libkq.so``.  It always recompiles.  Packed FP32
instructions are disabled for the device code (``-packed-fp32-ops``); hipcc's
host pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkq.so")
SOURCES = ["kq_kernels.hip", "kq_small_m.hip", "kq_abi.cpp"]
ARCH = "gfx950"


def _git_sha() -> str:
    try:
        out = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short", "HEAD"],
                             capture_output=True, text=True, timeout=10)
        return out.stdout.strip() or "unknown"
    except Exception:
        return "unknown"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found")


def flags() -> list[str]:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", f'-DKQ_GIT_SHA="{_git_sha()}"', "-I", os.path.join(ROOT, "include")]


def build(out: str = LIB, verbose: bool = False) -> str:
    tmp = out + f".tmp{os.getpid()}"
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [hipcc(), *flags(), "-shared", "-o", tmp, *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


def asm(source: str = "kq_kernels.hip", out_dir: str | None = None) -> str:
    """Write the gfx950 assembly of one source (for inspection) into out_dir,
    by default a new temporary directory; returns the file's path."""
    import tempfile
    out_dir = out_dir or tempfile.mkdtemp(prefix="kq_asm_")
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, os.path.splitext(source)[0] + ".s")
    cmd = [hipcc(), *flags(), "--cuda-device-only", "-S", "-o", out, os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
