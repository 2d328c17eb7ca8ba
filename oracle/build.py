"""Build the C oracle into oracle/liboracle.so with gcc.

Test infrastructure only: the product library never loads this.  Flags keep every
float operation a single IEEE-754 operation in program order: -O2 -ffp-contract=off,
no fast-math, SSE arithmetic (x86-64 default), C99.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "svdq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
