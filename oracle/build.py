"""Build the CPU oracle shared library (test infrastructure only).

Plain C99 compiled with gcc; -fno-fast-math and -ffp-contract=off keep every
FP32 product and sum separately rounded, as the oracle's definitions require.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "oracle.c")
CFLAGS = ["-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it; returns the library path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
