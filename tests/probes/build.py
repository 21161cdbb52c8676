"""Builds the test-only probe library (tests/probes/libprobes.so) for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libprobes.so")


def build() -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                    "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    os.path.join(HERE, "probes.hip"), "-o", tmp], check=True,
                   capture_output=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
