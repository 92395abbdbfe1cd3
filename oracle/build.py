"""Compile the CPU oracle (plain C) into ``oracle/libpeg_oracle.so``.

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg load the result. Flags keep it a plain scalar build:
no FMA contraction, no auto-vectorisation, no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "peg_oracle.c")
LIB = os.path.join(HERE, "libpeg_oracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-tree-vectorize", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(extra_flags=(), out=LIB):
    """Compile the oracle with gcc; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, *extra_flags, SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(out + ".tmp", out)
    return out


def ensure_built():
    """Build if the library is missing or older than its source."""
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(
            os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "peg_oracle.h"))):
        build()
    return LIB


if __name__ == "__main__":
    print(build())
