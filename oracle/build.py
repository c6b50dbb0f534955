"""Compile the C part of the oracle (test infrastructure only) with gcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "candidates.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Build oracle/liboracle.so from candidates.c; returns the library path."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, SRC],
                       check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
