"""Compile the device fill of the synthetic key/value generator."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "dpsynth_fill.hip")
LIB = os.path.join(HERE, "libdpsynth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "--offload-arch=gfx950", "-shared", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.run([HIPCC, *FLAGS, "-o", tmp, SRC], check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
