"""Build the CPU oracle (plain C, gcc, OpenMP) into oracle/_build/liboracle.so.

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg load the result; the HIP product library never does.
The flags keep binary64 arithmetic literal: no fast-math and no FMA
contraction, so every multiply and add rounds as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "liboracle.so")

CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11"]


def build(src=SRC, out=LIB, quiet=False):
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", *CFLAGS, src, "-o", out + ".tmp", "-lm"]
    if not quiet:
        print("[oracle] " + " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(quiet="-q" in sys.argv)
