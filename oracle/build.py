"""Compile the C oracle into ``oracle/liboracle.so`` with gcc (OpenMP, -O2).

Test infrastructure: the library it builds is loaded only by the tests, the smoke
check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Werror",
           *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]) if len(sys.argv) > 1 else build())
