"""Builds libmigemm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled separately (in parallel) into ``_build/`` and linked
into ``libmigemm.so`` next to this file.  Flags:

* ``--offload-arch=gfx950``: MI355X only, no other targets;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed FP32
  instructions in the device code (hipcc's host pass warns that it does not
  know the feature; the device pass honours it);
* ``-Rpass-analysis=kernel-resource-usage`` (optional): per-kernel VGPR, AGPR,
  LDS and scratch use, written to ``_build/resource_usage.txt``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmigemm.so")
# the two FP16/BF16 units first: they take longest
SOURCES = ["mfma16.hip", "mfma16_general.hip", "mfma_i8.hip", "api.cpp", "naive.hip", "lds_tiled.hip",
           "regtile_valu.hip", "regtile_mfma.hip", "fill.hip", "convert.hip", "pack.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, resource_usage: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    p = subprocess.run(cmd, capture_output=True, text=True)
    log = p.stdout + p.stderr
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{log}")
    return obj, log


def build(resource_usage: bool = False, jobs: int | None = None) -> str:
    """Compile all sources and link libmigemm.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_usage), SOURCES))
    if resource_usage:
        with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
            for src, (_, log) in zip(SOURCES, results):
                f.write(f"==== {src}\n")
                f.write("\n".join(l for l in log.splitlines() if "remark:" in l) + "\n")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *[obj for obj, _ in results]]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}{p.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv))
