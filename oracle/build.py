"""Compile the C oracle into oracle/liboracle_dp.so (test infrastructure).

gcc, -O2, no fused multiply-add contraction, no fast-math, OpenMP for the
layer/row loops.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dp_oracle.c")
LIB = os.path.join(HERE, "liboracle_dp.so")

FLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
         "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *FLAGS, "-o", tmp, SRC, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
