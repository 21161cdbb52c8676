"""GPU parity on the benchmark workloads, in the launch configuration the benchmark
times (migemm_gemm's own selection), against the CPU oracle.

Workloads up to 2050 x 2047 x 2056 are compared in full.  At 8192^3 (BF16) and
4096^3 (FP32) the oracle evaluates sampled entries one dot product each (random
positions, the four corners) plus whole blocks of rows and columns at the
matrix edges, which cover the edge tiles.
"""
import numpy as np
import pytest
import torch

import dense_gemm_16_amd as mg
import oracle
from oracle.check import compare, tolerance
from dense_gemm_16_amd import inputs
from gpu_helpers import check, run_gemm, sampled_entries, say, DT_CODE

pytestmark = pytest.mark.gpu

FULL = ["c0-f16-256", "c1-f32-1024", "c1-f32-1024-int", "c2-f16-1024", "c3-f16-2048",
        "c3-bf16-2048", "c3r-f16-2050x2047x2056"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_compare(name):
    w = inputs.WORKLOADS[name]
    A, B = w.make()
    say(f"workload {name} (selected path)")
    C, _ = run_gemm(A, B, w.dtype)
    check(C, A, B, w.dtype, exact=w.exact)


@pytest.mark.parametrize("name", ["c4-bf16-8192", "c4f-f32-4096", "s8-bf16-1024x8192x8192",
                                  "s2x4-bf16-4096x2048x8192"])
def test_workload_large_sampled(name):
    w = inputs.WORKLOADS[name]
    A, B = w.make()
    say(f"workload {name} (selected path, sampled check)")
    dA, dB = A.cuda(), B.cuda()
    C = torch.full((w.M, w.N), float("nan"), dtype=torch.float32, device="cuda")
    st = mg.migemm_gemm(w.M, w.N, w.K, DT_CODE[w.dtype], dA.data_ptr(), w.K, dB.data_ptr(), w.N,
                        C.data_ptr(), w.N, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mg.OK
    Ch = C.cpu()
    assert not torch.isnan(Ch).any(), "unwritten outputs"
    tol = tolerance(DT_CODE[w.dtype])
    bA, bB = inputs.to_bits(A), inputs.to_bits(B)
    rows, cols = sampled_entries(w.M, w.N, 3000, seed=1)
    ref, S = oracle.gemm_entries(bA, bB, DT_CODE[w.dtype], rows, cols)
    r = compare(Ch.numpy()[rows, cols], ref, S, tol=tol)
    assert r.ok, "sampled: " + str(r)
    # last 16 rows (bottom edge tiles), first 16 rows
    for r0 in (0, w.M - 16):
        ref, S = oracle.gemm(bA[r0:r0 + 16], bB, DT_CODE[w.dtype])
        r = compare(Ch.numpy()[r0:r0 + 16], ref, S, tol=tol)
        assert r.ok, f"rows {r0}..: " + str(r)
    # last 16 columns (right edge tiles)
    ref, S = oracle.gemm(bA, np.ascontiguousarray(bB[:, w.N - 16:]), DT_CODE[w.dtype])
    r = compare(Ch.numpy()[:, w.N - 16:], ref, S, tol=tol)
    assert r.ok, "last columns: " + str(r)
