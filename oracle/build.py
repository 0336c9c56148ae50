"""Build the oracle's shared library (plain C, gcc, OpenMP).

TEST INFRASTRUCTURE: the oracle is built so the tests, the smoke check and
the benchmark's CPU-baseline leg can call it; nothing in the product path
loads it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add, so each float operation in the
# oracle rounds once, as written.  No -ffast-math.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` into `out`; returns the output path."""
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
