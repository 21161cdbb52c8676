"""GPU parity on the benchmark workloads, in the launch configuration the benchmark
times (migemm_gemm's own selection), against the CPU oracle.

Workloads up to 2050 x 2047 x 2056, and the long-K and unaligned INT8 and FP32 ones, are compared in full here; the 8192^3,
4096^3 and one-GPU-share workloads in test_gpu_fullsize.py, also in full.
"""
import numpy as np
import pytest

from dense_gemm_16_amd import inputs
from gpu_helpers import check, run_gemm, say

pytestmark = pytest.mark.gpu

FULL = ["c0-f16-256", "c1-f32-1024", "c1-f32-1024-int", "c2-f16-1024", "c3-f16-2048",
        "c3-bf16-2048", "c3r-f16-2050x2047x2056", "lk-bf16-512x512x65536",
        "lk-f32-512x512x16384", "i8u-1000", "f32u-2049"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_compare(name):
    w = inputs.WORKLOADS[name]
    A, B = w.make()
    say(f"workload {name} (selected path)")
    if w.dtype == "i8":  # exact INT32 sums, the selection with the workspace it asks for
        from test_gpu_int8 import _want, run_i8
        C, intact = run_i8(A, B, ws=True)
        assert intact and np.array_equal(C, _want(A, B))
        return
    C, _ = run_gemm(A, B, w.dtype)
    check(C, A, B, w.dtype, exact=w.exact)
