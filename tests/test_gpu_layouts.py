"""Operands given transposed (MIGEMM_OP_T): A stored K x M, B stored N x K.

The product is the same C = A x B; only where the operands come from changes.
The oracle multiplies the row-major operands (the tests store their transposes
on the GPU), so every case here is the plain definition checked against a GPU
result computed from transposed storage: each variant and configuration, the
direct-staged kernels compiled for these layouts (and the register-staged
fallback for the others), padded and misaligned storage, the automatic
selection (the full 8192^3 BF16 shape in every layout is compared element by
element in test_gpu_fullsize.py).
"""
import pytest
import torch

import dense_gemm_16_amd as mg
from dense_gemm_16_amd import inputs
from gpu_helpers import check_ex, oracle_ref, padding_untouched, run_gemm_ex, say

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, True), (True, False), (True, True)]  # NT, TN, TT


def _name(ta, tb):
    return ("T" if ta else "N") + ("T" if tb else "N")


def _cases(dtype):
    code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    out = []
    for v in range(mg.migemm_variant_count()):
        if mg.migemm_variant_supports(v, code):
            out += [(v, c) for c in range(mg.migemm_config_count(v))]
    return out


# ragged; and one the direct-staged kernels take in every layout (M, N multiples
# of 8, K a multiple of 64)
SHAPES = [(97, 130, 200), (264, 296, 128)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_every_config_transposed_operands(dtype, ta, tb):
    for (M, N, K) in SHAPES:
        A, B = inputs.pair(M, N, K, dtype, "uniform", seed=M + 3 * N + K + 7 * ta + 11 * tb)
        ref = oracle_ref(A, B, dtype)
        for v, c in _cases(dtype):
            say(f"layout {_name(ta, tb)} {dtype} {M}x{N}x{K} variant={mg.migemm_variant_name(v)} cfg={c}")
            C, buf, mask = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None, variant=v, config=c,
                                       ta=ta, tb=tb)
            check_ex(C, A, B, dtype, 1.0, 0.0, 0, None, ref=ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_auto_selection_transposed(dtype, ta, tb):
    """The selected kernels (direct-staged where the shape allows, else register-
    staged) with a scaled update and 16-bit output as well."""
    for (M, N, K) in [(1, 1, 1), (512, 384, 256), (1000, 1032, 640), (1024, 1024, 1024)]:
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=M + N + K)
        ref = oracle_ref(A, B, dtype)
        say(f"layout auto {_name(ta, tb)} {dtype} {M}x{N}x{K}")
        C, _, _ = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None, ta=ta, tb=tb)
        check_ex(C, A, B, dtype, 1.0, 0.0, 0, None, ref=ref)
        old = (torch.rand((M, N), generator=torch.Generator().manual_seed(M)) - 0.5).to(torch.bfloat16)
        C, buf, mask = run_gemm_ex(A, B, dtype, -2.0, 0.5, 2, old, ta=ta, tb=tb)
        check_ex(C, A, B, dtype, -2.0, 0.5, 2, old, ref=ref)
        assert padding_untouched(buf, mask)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_integer_inputs_exact_transposed(ta, tb):
    M, N, K = 200, 136, 320
    for dtype in ("f32", "f16", "bf16"):
        A, B = inputs.pair(M, N, K, dtype, "int", seed=5 + ta + 2 * tb)
        ref = oracle_ref(A, B, dtype)
        for v, c in [(-1, -1)] + _cases(dtype):
            say(f"layout int {_name(ta, tb)} {dtype} variant={v} cfg={c}")
            C, _, _ = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None, variant=v, config=c, ta=ta,
                                  tb=tb)
            check_ex(C, A, B, dtype, 1.0, 0.0, 0, None, ref=ref, exact=True)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_padded_and_misaligned_transposed(ta, tb):
    """Stored operands with padded row strides (still multiples of 8: the direct
    path) and with a start 1 element into the allocation (the guarded path)."""
    M, N, K = 256, 264, 192
    for dtype in ("f32", "bf16"):
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=17)
        ref = oracle_ref(A, B, dtype)
        lda = (M if ta else K) + 24
        ldb = (K if tb else N) + 8
        for off in (0, 1):
            for v, c in [(-1, -1)] + _cases(dtype)[-3:]:
                say(f"layout padded {_name(ta, tb)} {dtype} off={off} variant={v} cfg={c}")
                C, _, _ = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None, variant=v, config=c,
                                      ta=ta, tb=tb, lda=lda, ldb=ldb, a_off=off, b_off=off)
                check_ex(C, A, B, dtype, 1.0, 0.0, 0, None, ref=ref)
