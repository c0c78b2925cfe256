"""Compile the CPU oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure only. The flags are deliberately plain: -O2 and no
-ffast-math, so that the compensation term of the compensated sum survives.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-pthread", "-Wall", "-Wextra", "-Werror"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` to the shared library `out`; return `out`."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(), file=sys.stderr)
