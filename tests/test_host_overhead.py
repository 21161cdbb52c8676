"""Host time of the entry checks and configuration selection (no GPU).

A product call validates its arguments and picks a configuration on the host
before it launches anything; for the small products (256^3, 1024^3) that runs
next to kernels of a few microseconds, so it has to stay well below one.
`host_overhead.c` times migemm_select (the checks and the selection table) and
migemm_workspace_size (plus the packed path's size rule) over aligned, ragged,
transposed, FP32, FP16, BF16 and INT8 shapes, linked against the built library.
"""
import os
import shutil
import subprocess

import pytest

import dense_gemm_16_amd as mg

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_selection_host_time_well_below_a_microsecond(tmp_path):
    lib_dir = os.path.dirname(mg.LIBRARY_PATH)
    exe = str(tmp_path / "host_overhead")
    subprocess.run(["gcc", "-O2", "-I", os.path.join(ROOT, "include"),
                    os.path.join(HERE, "host_overhead.c"), "-L", lib_dir, "-lmigemm",
                    f"-Wl,-rpath,{lib_dir}", "-o", exe], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    vals = dict(line.split() for line in out.splitlines())
    select_ns, ws_ns = float(vals["select_ns"]), float(vals["workspace_size_ns"])
    print(f"migemm_select {select_ns:.0f} ns, migemm_workspace_size {ws_ns:.0f} ns per call")
    assert select_ns < 500.0 and ws_ns < 500.0, out
