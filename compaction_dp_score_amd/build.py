"""Build libdecoprune.so in place with hipcc for gfx950."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdecoprune.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-shared", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(force: bool = True, extra=()) -> str:
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.run([HIPCC, *FLAGS, *extra, "-o", tmp, *sources()], check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
