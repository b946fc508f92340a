"""Build the fp64 oracle (plain C, OpenMP) into oracle/liboracle.so.

Test infrastructure: see oracle/__init__.py for who may load it.
Usage: python -m oracle.build   (or call build()).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No fast-math and no contraction: the oracle's rounding follows the source order.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra"]


def build(extra_flags=(), src: str = SRC, out: str = LIB, quiet: bool = True) -> str:
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(out + ".tmp", out)
    return out


def stale() -> bool:
    return (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC)


if __name__ == "__main__":
    print(build(quiet=False))
