"""GPU parity at the full benchmark sizes: every element of C against the CPU
oracle, in the launch configurations the benchmark times (the library's own
selection).

* 8192^3 BF16 (the headline): one oracle pass (C_ref and the tolerance scale S
  over the same rounded inputs) serves the four operand layouts (A and B stored
  as given or transposed) and the general output step (C = 0.5 A B - 1.0 C_old
  stored as BF16);
* 4096^3 FP32, and one GPU's share of an 8-way split of the headline
  (1024 x 8192 x 8192 and 4096 x 2048 x 8192 BF16), each against its own
  oracle pass;
* 8192^3 INT8 -> INT32, bit-exact.

At these sizes the product runs many rounds of workgroups per CU (4 for the
headline's 1024 tiles of 256 x 256), so every tile position, round and edge is
covered; a NaN-filled C shows any element left unwritten.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_gemm_16_amd import inputs
from gpu_helpers import check_ex, oracle_ref, run_gemm_ex, say
from test_gpu_int8 import run_i8

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


@pytest.fixture(scope="module")
def headline():
    w = inputs.WORKLOADS["c4-bf16-8192"]
    A, B = w.make()
    say(f"oracle {w.name}: one pass over {w.M}x{w.N}x{w.K} on {oracle.threads_used()} threads")
    ref = oracle_ref(A, B, w.dtype)
    return w, A, B, ref


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_headline_full_every_layout(headline, ta, tb):
    w, A, B, ref = headline
    name = ("T" if ta else "N") + ("T" if tb else "N")
    say(f"{w.name} layout {name}: every element")
    C, _, _ = run_gemm_ex(A, B, w.dtype, 1.0, 0.0, 0, None, ta=ta, tb=tb)
    assert not torch.isnan(C).any(), "unwritten outputs"
    r = check_ex(C, A, B, w.dtype, 1.0, 0.0, 0, None, ref=ref)
    say(f"  {r}")


def test_headline_full_general_output_bf16(headline):
    w, A, B, ref = headline
    old = torch.randn((w.M, w.N), generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    say(f"{w.name} C = 0.5 A B - 1.0 C_old, BF16 C: every element")
    C, _, _ = run_gemm_ex(A, B, w.dtype, 0.5, -1.0, 2, old)
    r = check_ex(C, A, B, w.dtype, 0.5, -1.0, 2, old, ref=ref)
    say(f"  {r}")


@pytest.mark.parametrize("name", ["c4f-f32-4096", "s8-bf16-1024x8192x8192",
                                  "s2x4-bf16-4096x2048x8192"])
def test_large_full(name):
    w = inputs.WORKLOADS[name]
    A, B = w.make()
    say(f"{name}: every element")
    C, _, _ = run_gemm_ex(A, B, w.dtype, 1.0, 0.0, 0, None)
    assert not torch.isnan(C).any(), "unwritten outputs"
    r = check_ex(C, A, B, w.dtype, 1.0, 0.0, 0, None)
    say(f"  {r}")


def test_int8_headline_full_exact():
    w = inputs.WORKLOADS["i8-8192"]
    A, B = w.make()
    say(f"{w.name}: every element, exact")
    C, intact = run_i8(A, B)
    assert intact
    say(f"oracle {w.name} on {oracle.threads_used()} threads")
    want, _ = oracle.gemm(A.numpy(), B.numpy(), oracle.I8, want_scale=False)
    bad = np.argwhere(C.astype(np.float64) != want)
    assert bad.size == 0, (f"{len(bad)} mismatches, first at {tuple(bad[0])}: "
                           f"got {C[tuple(bad[0])]}, want {want[tuple(bad[0])]}")
