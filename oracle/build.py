"""Compile the CPU oracle (test infrastructure) into oracle/liborr_oracle.so.

Flags keep every float operation a single IEEE single-precision operation
rounded to nearest, in source order: no contraction into fused multiply-add,
no fast-math reassociation, x86-64 SSE arithmetic (no extended precision).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "orr_oracle.c")
LIB = os.path.join(HERE, "liborr_oracle.so")

FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-fno-math-errno", "-mfpmath=sse", "-Wall", "-Wextra"]


def build(extra_flags=(), out=LIB) -> str:
    cmd = ["gcc", *FLAGS, *extra_flags, SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
