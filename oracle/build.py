"""Build the CPU oracle library (test infrastructure) with gcc.

``build()`` writes ``oracle/liboracle.so``; ``build(plant=n)`` writes a copy
with one deliberate mistake compiled in (``liboracle_plant<n>.so``) for the
tests that show the pins catch mistakes.  IEEE binary64 semantics are kept:
no fast-math, no contraction of multiply-add pairs.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kq_oracle.c")


def lib_path(plant: int = 0) -> str:
    name = "liboracle.so" if plant == 0 else f"liboracle_plant{plant}.so"
    return os.path.join(HERE, name)


def build(plant: int = 0, out: str | None = None) -> str:
    out = out or lib_path(plant)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", f"-DORC_PLANT={int(plant)}", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
