"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

The oracle is test infrastructure: building it is part of the build check,
using it is reserved to the tests, the smoke check and the bench's CPU
baseline.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


def build(extra=(), out=OUT):
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
