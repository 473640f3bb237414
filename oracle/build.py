"""Builds the oracle's shared library (test infrastructure only).

Compiled with gcc, no fast-math and no FMA contraction, so that every fp32
step in oracle.c is a single IEEE operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fno-finite-math-only", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
