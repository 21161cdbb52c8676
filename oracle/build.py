"""Builds the oracle's C library with the host compiler (test infrastructure only)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile oracle.c into liboracle.so next to it and return the path.

    -ffp-contract=off keeps every binary64 multiply and add separately rounded;
    no -march flag, so the library runs on any x86-64 host.
    """
    src = os.path.join(_HERE, "oracle.c")
    out = library_path()
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-shared", "-fPIC", src, "-lm", "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
