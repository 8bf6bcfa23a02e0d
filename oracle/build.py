"""Compile the oracle's C part (csa.c) into oracle/_csa.so with gcc.

Flags: -O2 -ffp-contract=off (no fused multiply-add unless fmaf() is written),
no fast-math, SSE2 binary32 arithmetic on x86-64 (no excess precision)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csa.c")
OUT = os.path.join(HERE, "_csa.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(OUT) and os.path.getmtime(OUT) >= os.path.getmtime(SRC):
        return OUT
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra",
           "-o", OUT + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(force="--force" in sys.argv or True))
