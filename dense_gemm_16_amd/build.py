"""Builds libmigemm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled separately (in parallel) into ``_build/`` and linked
into ``libmigemm.so`` next to this file.  Flags:

* ``--offload-arch=gfx950``: MI355X only, no other targets;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed FP32
  instructions in the device code (hipcc's host pass warns that it does not
  know the feature; the device pass honours it);
* ``-Rpass-analysis=kernel-resource-usage``: the compiler's per-kernel SGPR,
  VGPR, AGPR, scratch, spill, LDS and occupancy figures, collected into
  ``kernel_resources.json`` next to the library (keyed by the kernel's symbol,
  with its demangled name), which the benchmark reports per timed kernel.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmigemm.so")
RESOURCES = os.path.join(PKG, "kernel_resources.json")
SOURCES = ["api.cpp", "mfma16.hip", "mfma_i8.hip", "regtile_mfma.hip", "naive.hip",
           "lds_tiled.hip", "regtile_valu.hip", "fill.hip", "convert.hip", "pack.hip",
           "noalloc.hip", "skinny.hip", "split.cpp", "splitk.hip"]
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
          for gen in (False, True) for c in range(12)] +
         [("mfma_i8_part.hip", f"mfma_i8_{c}", [f"-DMIGEMM_PART_C={c}"]) for c in (0, 1, 2, 3, 4, 6)])
# Units that take longest, started first (measured compile times, seconds).
SLOW_FIRST = ("mfma16_f16_gen_14", "mfma16_bf16_gen_14", "mfma_i8_4", "mfma16_f16_gen_4",
              "mfma16_f16_gen_15", "mfma16_f16_gen_1", "mfma16_bf16_gen_15",
              "mfma16_f16_plain_14", "mfma16_bf16_gen_1", "mfma16_f16_gen_0",
              "mfma16_bf16_plain_14", "mfma16_bf16_gen_0", "mfma16_bf16_gen_4")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(job, force: bool) -> str:
    src, name, defines = job
    obj = os.path.join(BUILD, name + ".o")
    res = os.path.join(BUILD, name + ".res.json")
    if not force and _up_to_date(obj, os.path.join(CSRC, src)) and os.path.exists(res):
        return obj
    cmd = [HIPCC, "-Rpass-analysis=kernel-resource-usage", *FLAGS, *defines, "-c",
           os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    log = p.stdout + p.stderr
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} ({name}):\n{log}")
    with open(res, "w") as f:
        json.dump(_parse_remarks(log), f)
    return obj


_FIELDS = {"TotalSGPRs": "sgpr", "VGPRs": "vgpr", "AGPRs": "agpr",
           "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
           "Occupancy [waves/SIMD]": "occupancy_waves_per_simd", "SGPRs Spill": "sgpr_spill",
           "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds_bytes"}


def _parse_remarks(log: str) -> dict:
    """Per-kernel figures from the kernel-resource-usage remarks of one compile."""
    out, cur = {}, None
    for line in log.splitlines():
        m = re.search(r"remark: (?:Function Name: (\S+)|\s+([^:]+): (\S+))", line)
        if not m or "kernel-resource-usage" not in line:
            continue
        if m.group(1):
            cur = out.setdefault(m.group(1), {})
        elif cur is not None and m.group(2).strip() in _FIELDS:
            v = m.group(3)
            cur[_FIELDS[m.group(2).strip()]] = int(v) if v.isdigit() else v
    return out


def _write_resources(objs) -> None:
    """Merges the per-object remark figures into kernel_resources.json, with
    demangled names (c++filt, where present)."""
    table = {}
    for obj in objs:
        try:
            with open(os.path.splitext(obj)[0] + ".res.json") as f:
                table.update(json.load(f))
        except (OSError, ValueError):
            pass
    names = sorted(table)
    try:
        p = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True,
                           check=True)
        demangled = p.stdout.splitlines()
    except (OSError, subprocess.CalledProcessError):
        demangled = []
    if len(demangled) == len(names):
        for n, d in zip(names, demangled):
            table[n]["demangled"] = d
    with open(RESOURCES, "w") as f:
        json.dump({"note": "compiler figures per kernel (-Rpass-analysis=kernel-resource-usage)",
                   "kernels": table}, f, indent=0)


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


def build(jobs: int | None = None, force: bool = True) -> str:
    """Compile all sources and link libmigemm.so; returns the library path.

    force=False recompiles only objects older than their source or any header."""
    os.makedirs(BUILD, exist_ok=True)
    us = units()
    jobs = jobs or max(1, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, force), us))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}{p.stderr}")
    os.replace(tmp, LIB)
    _write_resources(objs)
    return LIB


if __name__ == "__main__":
    print(build(force="--incremental" not in sys.argv))
