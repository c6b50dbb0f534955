"""Compile the C part of the oracle (test infrastructure only) with gcc: the candidate
build (candidates.c) and the loss and gradients (ce.c, OpenMP over token blocks)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(HERE, "candidates.c"), os.path.join(HERE, "ce.c")]
SRC = SOURCES[0]
LIB = os.path.join(HERE, "liboracle.so")
# x86-64-v3 (AVX2, FMA) runs on every host CPU these GPUs are paired with; the flags
# only change speed and the rounding order of the double-precision dot products
FLAGS = ["-O3", "-march=x86-64-v3", "-fopenmp", "-Wall", "-Wextra", "-shared", "-fPIC"]


def stale() -> bool:
    return not os.path.exists(LIB) or any(os.path.getmtime(LIB) < os.path.getmtime(s)
                                          for s in SOURCES)


def build(force: bool = True) -> str:
    """Build oracle/liboracle.so from the C sources; returns the library path."""
    if force or stale():
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", *FLAGS, "-o", tmp, *SOURCES, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
