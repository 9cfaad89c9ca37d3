"""Compile the CPU oracle (plain C11, host only) into oracle/libkgref.so.

Test infrastructure: building the checker is not using it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkgref.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "kgref.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
