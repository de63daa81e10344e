"""Compile the oracle's C helper with gcc (test infrastructure only).

Builds ``oracle/_build/liboracle_logits.so`` from ``fixed_order_logits.c``.
The flags keep IEEE float32 semantics: no fast-math, no contraction of the
separate bias add, and math-errno off only so that ``fmaf`` can be inlined.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fixed_order_logits.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "liboracle_logits.so")

CFLAGS = ["-O3", "-fno-math-errno", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-std=c11"]


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
