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
SOURCES = ["api.cpp", "mfma16.hip", "mfma_i8.hip", "regtile_mfma.hip", "naive.hip",
           "lds_tiled.hip", "regtile_valu.hip", "fill.hip", "convert.hip", "pack.hip"]
# The configuration tables' kernels are built from *_part.hip sources, once per
# configuration (and element type and output form), so that the compiles run in
# parallel and a change rebuilds only what it touches.
CFG16 = [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 13, 14, 15, 16]
PARTS = ([("mfma16_part.hip", f"mfma16_{et}_{'gen' if gen else 'plain'}_{c}",
           [f"-DMIGEMM_PART_E={e}", f"-DMIGEMM_PART_GEN={'true' if gen else 'false'}",
            f"-DMIGEMM_PART_C={c}"])
          for et, e in (("f16", "_Float16"), ("bf16", "bf16_t"))
          for gen in (False, True) for c in CFG16] +
         [("regtile_mfma_part.hip", f"regtile_mfma_{'gen' if gen else 'plain'}_{c}",
           [f"-DMIGEMM_PART_GEN={'true' if gen else 'false'}", f"-DMIGEMM_PART_C={c}"])
          for gen in (False, True) for c in range(8)] +
         [("mfma_i8_part.hip", f"mfma_i8_{c}", [f"-DMIGEMM_PART_C={c}"]) for c in range(5)])
# Units that take longest, started first (measured compile times, seconds).
SLOW_FIRST = ("mfma16_f16_gen_14", "mfma16_bf16_gen_14", "mfma_i8_4", "mfma16_f16_gen_4",
              "mfma16_f16_gen_15", "mfma16_f16_gen_1", "mfma16_bf16_gen_15",
              "mfma16_f16_plain_14", "mfma16_bf16_gen_1", "mfma16_f16_gen_0",
              "mfma16_bf16_plain_14", "mfma16_bf16_gen_0", "mfma16_bf16_gen_4")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(job, resource_usage: bool, force: bool) -> tuple[str, str]:
    src, name, defines = job
    obj = os.path.join(BUILD, name + ".o")
    if not force and not resource_usage and _up_to_date(obj, os.path.join(CSRC, src)):
        return obj, ""
    cmd = [HIPCC, *FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    p = subprocess.run(cmd, capture_output=True, text=True)
    log = p.stdout + p.stderr
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} ({name}):\n{log}")
    return obj, log


def _up_to_date(obj: str, src: str) -> bool:
    """The object is newer than its source, every header, this script and the flags."""
    try:
        t = os.path.getmtime(obj)
    except OSError:
        return False
    deps = [src, os.path.abspath(__file__), os.path.join(ROOT, "include", "migemm.h")]
    deps += [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    return all(os.path.getmtime(d) < t for d in deps)


def units():
    """(source, object name, defines) of every compile, slowest first."""
    u = PARTS + [(src, os.path.splitext(src)[0], []) for src in SOURCES]
    rank = {n: i for i, n in enumerate(SLOW_FIRST)}
    return sorted(u, key=lambda x: rank.get(x[1], len(rank)))


def build(resource_usage: bool = False, jobs: int | None = None, force: bool = True) -> str:
    """Compile all sources and link libmigemm.so; returns the library path.

    force=False recompiles only objects older than their source or any header."""
    os.makedirs(BUILD, exist_ok=True)
    us = units()
    jobs = jobs or max(1, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda u: _compile(u, resource_usage, force), us))
    if resource_usage:
        with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
            for (_, name, _), (_, log) in zip(us, results):
                f.write(f"==== {name}\n")
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
    print(build(resource_usage="--resource-usage" in sys.argv, force="--incremental" not in sys.argv))
