"""The general output step on the GPU: C = alpha * A x B + beta * C_old, with C
stored as FP32, FP16 or BF16, against the oracle's update
(``oracle.epilogue``) and its round-to-nearest-even encoder (``oracle.encode``).

The sum of products is the same FP32 accumulation the plain tests cover; here
the checks add the scaled update, the final rounding (exact where the exact
result is known: ties, overflow, integers), that the previous C is not read
when beta == 0, and that nothing outside the M x N window of C is written.
"""
import numpy as np
import pytest
import torch

import dense_gemm_16_amd as mg
import oracle
from dense_gemm_16_amd import inputs
from gpu_helpers import (TORCH_OF, check_ex, oracle_ref, padding_untouched, run_gemm_ex, say)

pytestmark = pytest.mark.gpu

C_CODES = [0, 1, 2]


def _cases(dtype):
    code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    out = []
    for v in range(mg.migemm_variant_count()):
        if mg.migemm_variant_supports(v, code):
            out += [(v, c) for c in range(mg.migemm_config_count(v))]
    return out


def _old(M, N, c_code, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.rand((M, N), generator=g) * 4 - 2).to(TORCH_OF[c_code])


# a ragged shape that no tile divides, and one the direct-staged kernels take
# (K a multiple of 64, N a multiple of 8, rows of A and B in whole 16-byte chunks)
SHAPES = [(97, 130, 200), (300, 264, 128)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_every_config_general_update(dtype):
    for (M, N, K) in SHAPES:
        A, B = inputs.pair(M, N, K, dtype, "uniform", seed=M + 5 * N + K)
        ref = oracle_ref(A, B, dtype)
        for c_code in C_CODES:
            old = _old(M, N, c_code, seed=M + c_code)
            for v, c in _cases(dtype):
                say(f"general {dtype} {M}x{N}x{K} out={c_code} variant={mg.migemm_variant_name(v)} cfg={c}")
                C, buf, mask = run_gemm_ex(A, B, dtype, 1.5, -0.75, c_code, old, variant=v,
                                           config=c)
                check_ex(C, A, B, dtype, 1.5, -0.75, c_code, old, ref=ref)
                assert padding_untouched(buf, mask)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_every_config_general_update_whole_line_rows(dtype):
    """Rows of C that start whole 128-byte lines (N = 512 for FP32 and 16-bit C):
    the configurations that pick their store policy by C's layout take the
    non-temporal one here, the shapes above take plain stores."""
    M, N, K = 256, 512, 192
    A, B = inputs.pair(M, N, K, dtype, "uniform", seed=41)
    ref = oracle_ref(A, B, dtype)
    for c_code in C_CODES:
        old = _old(M, N, c_code, seed=43 + c_code)
        for v, c in _cases(dtype):
            say(f"general whole-line {dtype} {M}x{N}x{K} out={c_code} "
                f"variant={mg.migemm_variant_name(v)} cfg={c}")
            C, buf, mask = run_gemm_ex(A, B, dtype, 1.5, -0.75, c_code, old, variant=v, config=c)
            check_ex(C, A, B, dtype, 1.5, -0.75, c_code, old, ref=ref)
            assert padding_untouched(buf, mask)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("c_code", C_CODES)
def test_auto_selection_general_update(dtype, c_code):
    for (M, N, K) in [(1, 1, 1), (64, 64, 64), (513, 776, 256), (1000, 520, 640)]:
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=3 * M + N + K + c_code)
        old = _old(M, N, c_code, seed=K)
        say(f"general auto {dtype} {M}x{N}x{K} out={c_code}")
        C, buf, mask = run_gemm_ex(A, B, dtype, -0.5, 2.0, c_code, old)
        check_ex(C, A, B, dtype, -0.5, 2.0, c_code, old)
        assert padding_untouched(buf, mask)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("c_code", C_CODES)
def test_beta_zero_leaves_previous_c_unread(dtype, c_code):
    """The window starts as NaN; with beta == 0 the result has no NaN."""
    M, N, K = 300, 264, 128
    A, B = inputs.pair(M, N, K, dtype, "uniform", seed=71)
    ref = oracle_ref(A, B, dtype)
    for v, c in [(-1, -1)] + [x for x in _cases(dtype) if x[0] == mg.NAIVE]:
        say(f"beta0 {dtype} out={c_code} variant={v} cfg={c}")
        C, buf, mask = run_gemm_ex(A, B, dtype, 3.0, 0.0, c_code, None, variant=v, config=c)
        assert not torch.isnan(C.float()).any()
        check_ex(C, A, B, dtype, 3.0, 0.0, c_code, None, ref=ref)


@pytest.mark.parametrize("c_code", C_CODES)
def test_integer_update_exact(c_code):
    """Small integers: the sum, the update and its rounding are all exact (results stay
    below 2^11, exact in FP16 and, here, in BF16's 8 bits as well: |C| <= 255)."""
    M, N, K = 70, 90, 6
    g = torch.Generator().manual_seed(13)
    for dtype in ("f32", "f16", "bf16"):
        A = torch.randint(-2, 3, (M, K), generator=g).float().to(inputs.TORCH_DTYPES[dtype])
        B = torch.randint(-2, 3, (K, N), generator=g).float().to(inputs.TORCH_DTYPES[dtype])
        old = torch.randint(-30, 31, (M, N), generator=g).float().to(TORCH_OF[c_code])
        for v, c in [(-1, -1)] + _cases(dtype)[:3]:
            say(f"int exact {dtype} out={c_code} variant={v} cfg={c}")
            C, _, _ = run_gemm_ex(A, B, dtype, 2.0, -3.0, c_code, old, variant=v, config=c)
            check_ex(C, A, B, dtype, 2.0, -3.0, c_code, old, exact=True)


def _midpoints(c_code, n, seed):
    """n values exactly halfway between adjacent values of the output format (and
    exact in FP32): the rounding must go to the even neighbour."""
    rng = np.random.default_rng(seed)
    if c_code == 1:
        lo = rng.integers(0x0400, 0x7BFF, n).astype(np.uint16)        # normal binary16
    else:
        lo = rng.integers(0x0080, 0x7F7F, n).astype(np.uint16) & 0x3FFF | 0x3000  # moderate bf16
    a = oracle.decode(lo, c_code)
    b = oracle.decode(lo + 1, c_code)
    mid = (a + b) / 2
    sign = np.where(rng.integers(0, 2, n) == 1, -1.0, 1.0)
    return (mid * sign).astype(np.float32)


@pytest.mark.parametrize("c_code", [1, 2])
def test_rounding_ties_to_even_bit_exact(c_code):
    """FP32 inputs, K = 1, A holds exact midpoints of the output format, B = 1: every
    variant's stored result must be the oracle's round-to-nearest-even encoding."""
    M = 512
    mids = _midpoints(c_code, M, seed=c_code)
    A = torch.from_numpy(mids).view(M, 1)
    B = torch.ones(1, 1)
    want = oracle.encode(mids.astype(np.float64), c_code)
    for v, c in [(-1, -1)] + _cases("f32"):
        say(f"ties out={c_code} variant={v} cfg={c}")
        C, _, _ = run_gemm_ex(A, B, "f32", 1.0, 0.0, c_code, None, variant=v, config=c)
        got = C.view(torch.int16).numpy().view(np.uint16).reshape(-1)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"{bad.size} differ; first row {bad[0]}: value {mids[bad[0]]!r} "
                               f"got {got[bad[0]]:#06x} want {want[bad[0]]:#06x}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rounding_ties_through_matrix_cores(dtype):
    """16-bit inputs on the matrix-core path: rows whose two products add up (exactly,
    in FP32) to a BF16 midpoint, stored as BF16 by the direct-staged and register-
    staged kernels: the even neighbour, bit for bit."""
    M, N, K = 256, 256, 64
    g = torch.Generator().manual_seed(29)
    # x + y with x in [1, 2) on the BF16 grid and y = 2^-8: the midpoint above x
    xs = 1.0 + torch.randint(0, 128, (M,), generator=g).float() / 128
    A = torch.zeros(M, K)
    A[:, 0] = xs
    A[:, 1] = 2.0 ** -8
    B = torch.zeros(K, N)
    B[0, :] = 1.0
    B[1, :] = 1.0
    A = A.to(inputs.TORCH_DTYPES[dtype])
    B = B.to(inputs.TORCH_DTYPES[dtype])
    exact = (xs.double() + 2.0 ** -8).numpy()
    want = np.repeat(oracle.encode(exact, 2)[:, None], N, axis=1)
    for v, c in [(-1, -1)] + [x for x in _cases(dtype) if x[0] == mg.MFMA16]:
        say(f"ties mfma {dtype} variant={v} cfg={c}")
        C, _, _ = run_gemm_ex(A, B, dtype, 1.0, 0.0, 2, None, variant=v, config=c)
        got = C.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("c_code", [1, 2])
def test_overflow_to_infinity(c_code):
    """Results beyond the output format's range become +-infinity (the oracle's
    encoding of the exact value), values just inside stay finite."""
    if c_code == 1:   # largest 65504, quantum 32: 65520 is the tie with 2^16
        vals = [65504.0, -65504.0, 65519.0, 65520.0, -65520.0, 70000.0, 1e30, 1.0]
    else:             # largest (2 - 2^-7) 2^127, quantum 2^120: + 2^119 is the tie with 2^128
        top = (2 - 2 ** -7) * 2.0 ** 127
        vals = [top, -top, top + 2.0 ** 118, top + 2.0 ** 119, -(top + 2.0 ** 119), 1.0]
    vals = np.array(vals, dtype=np.float32)
    assert np.isfinite(vals).all()
    A = torch.from_numpy(vals).view(-1, 1)
    B = torch.ones(1, 1)
    want = oracle.encode(vals.astype(np.float64), c_code)
    for v, c in [(-1, -1), (mg.NAIVE, 0)]:
        say(f"overflow out={c_code} variant={v}")
        C, _, _ = run_gemm_ex(A, B, "f32", 1.0, 0.0, c_code, None, variant=v, config=c)
        got = C.view(torch.int16).numpy().view(np.uint16).reshape(-1)
        assert np.array_equal(got, want), (got, want)


@pytest.mark.parametrize("c_code", C_CODES)
def test_empty_product_scales_previous_c(c_code):
    """K == 0: C = beta * C_old (rounded); with beta == 0, C = 0."""
    M, N = 33, 47
    old = _old(M, N, c_code, seed=3)
    A = torch.zeros(M, 0)
    B = torch.zeros(0, N)
    C, buf, mask = run_gemm_ex(A, B, "f32", 2.0, -1.5, c_code, old, ldc=64, c_off=3)
    zero = np.zeros((M, N))
    upd, _ = oracle.epilogue(zero, zero, 2.0, -1.5, c_code, inputs.to_bits(old))
    want = oracle.encode(upd, c_code)
    got = C.numpy() if c_code == 0 else C.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert padding_untouched(buf, mask)
    C, _, _ = run_gemm_ex(A, B, "f32", 2.0, 0.0, c_code, None)
    assert torch.all(C.float() == 0)


@pytest.mark.parametrize("c_code", [1, 2])
def test_padded_and_offset_output(c_code):
    """C with a padded row stride and a start 1 element into its allocation (2-byte
    aligned only): the window gets the update, the padding keeps its NaN."""
    M, N, K = 200, 136, 128
    for dtype in ("f32", "bf16"):
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=41)
        old = _old(M, N, c_code, seed=4)
        for v, c in [(-1, -1)] + _cases(dtype)[:4]:
            say(f"padded out={c_code} {dtype} variant={v} cfg={c}")
            C, buf, mask = run_gemm_ex(A, B, dtype, 0.75, 0.25, c_code, old, variant=v,
                                       config=c, ldc=N + 13, c_off=1)
            check_ex(C, A, B, dtype, 0.75, 0.25, c_code, old)
            assert padding_untouched(buf, mask)
