"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every test here runs on the CPU.  The oracle computes
C[i][j] = sum_k A[i][k] B[k][j] in binary64 (page "Tensor cores and matrix
operations", section "Traditional Approach: Element-by-Element").  It is checked
against: the decoders of torch (an independent implementation of the IEEE
binary16 and bfloat16 layouts) on all 65,536 patterns and a hand-written
table; a hand-worked product; closed forms (all-ones gives K, identity and
permutation give the other operand exactly); exact integer products from
numpy's int64 matmul; and exact rational brute force (fractions) on 4x4 and
16x16 inputs.  ``test_oracle_mutants.py`` shows that each of these would
catch a plausible mistake.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.check import compare, TOL_F32, TOL_HALF
from dense_gemm_16_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DT = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}


def bits(t):
    return inputs.to_bits(t)


# ---------------------------------------------------------------- decoders

@pytest.mark.parametrize("name,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_decode_exhaustive_matches_torch(name, tdt):
    allbits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(allbits, DT[name])
    want = torch.from_numpy(allbits.view(np.int16).copy()).view(tdt).double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros decode with their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_golden_table():
    n = 0
    with open(os.path.join(GOLDEN, "decode_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, hexbits, value = line.split()
            got = oracle.decode(np.array([int(hexbits, 16)], dtype=np.uint16), DT[name])[0]
            want = float(value)
            assert got == want and np.signbit(got) == np.signbit(want), (name, hexbits, got)
            n += 1
    assert n >= 19


def test_decode_f32_is_widening():
    x = np.array([1.5, -0.0, 3.4028234663852886e38, 1.401298464324817e-45, np.inf],
                 dtype=np.float32)
    assert np.array_equal(oracle.decode(x, oracle.F32), x.astype(np.float64))


# ------------------------------------------------------- hand-worked example

def _read_golden_matrices(path):
    mats, cur, rows = {}, None, 0
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            if parts[0].isalpha():
                cur, rows = parts[0], int(parts[1])
                mats[cur] = []
                continue
            mats[cur].append([float(v) for v in parts])
    return {k: np.array(v) for k, v in mats.items()}


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_textbook_example(dt):
    m = _read_golden_matrices(os.path.join(GOLDEN, "textbook_2x3x2.txt"))
    A = torch.tensor(m["A"], dtype=torch.float32).to(inputs.TORCH_DTYPES[dt])
    B = torch.tensor(m["B"], dtype=torch.float32).to(inputs.TORCH_DTYPES[dt])
    C, S = oracle.gemm(bits(A), bits(B), DT[dt])
    assert np.array_equal(C, m["C"])
    # all entries positive, so S equals C
    assert np.array_equal(S, m["C"])


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 9, 33), (4, 4, 0), (64, 48, 300)])
def test_all_ones_gives_K(dt, M, N, K):
    A = torch.ones(M, K).to(inputs.TORCH_DTYPES[dt])
    B = torch.ones(K, N).to(inputs.TORCH_DTYPES[dt])
    C, S = oracle.gemm(bits(A), bits(B), DT[dt])
    assert C.shape == (M, N)
    assert np.all(C == K) and np.all(S == K)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_identity_left_and_right(dt):
    n, p = 37, 23
    B = inputs.draw((n, p), dt, "normal", torch.Generator().manual_seed(5))
    I = torch.eye(n).to(inputs.TORCH_DTYPES[dt])
    C, _ = oracle.gemm(bits(I), bits(B), DT[dt])
    assert np.array_equal(C, B.double().numpy())
    A = inputs.draw((p, n), dt, "uniform", torch.Generator().manual_seed(6))
    C, _ = oracle.gemm(bits(A), bits(I), DT[dt])
    assert np.array_equal(C, A.double().numpy())


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_permutation_rows_and_columns(dt):
    n, p = 41, 19
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(7))
    P = torch.zeros(n, n)
    P[torch.arange(n), perm] = 1.0          # (P B)[i] = B[perm[i]]
    P = P.to(inputs.TORCH_DTYPES[dt])
    B = inputs.draw((n, p), dt, "normal", torch.Generator().manual_seed(8))
    C, _ = oracle.gemm(bits(P), bits(B), DT[dt])
    assert np.array_equal(C, B.double().numpy()[perm.numpy()])
    # right-multiplication permutes columns: (A P)[:, j] = A[:, q[j]] with P[q[j], j] = 1
    A = inputs.draw((p, n), dt, "normal", torch.Generator().manual_seed(9))
    C, _ = oracle.gemm(bits(A), bits(P), DT[dt])
    q = torch.argmax(P.float(), dim=0).numpy()
    assert np.array_equal(C, A.double().numpy()[:, q])


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(33, 65, 129), (128, 96, 1000)])
def test_small_integers_exact(dt, M, N, K):
    A, B = inputs.pair(M, N, K, dt, "int", seed=M + N + K)
    want = A.double().numpy().astype(np.int64) @ B.double().numpy().astype(np.int64)
    C, S = oracle.gemm(bits(A), bits(B), DT[dt])
    assert np.array_equal(C, want.astype(np.float64))
    wantS = np.abs(A.double().numpy().astype(np.int64)) @ np.abs(B.double().numpy().astype(np.int64))
    assert np.array_equal(S, wantS.astype(np.float64))


def test_page3_integer_pattern_exact():
    # the exact small-integer fill of page "matmul_registers.cu" (fillInputs)
    n = 96
    A, B = inputs.pair(n, n, n, "f32", "p3", seed=0)
    r = np.arange(n).reshape(-1, 1)
    c = np.arange(n).reshape(1, -1)
    a = ((r + 2 * c) % 7) - 3
    b = ((3 * r + c) % 5) - 2
    assert np.array_equal(A.numpy(), a.astype(np.float32))
    C, _ = oracle.gemm(bits(A), bits(B), oracle.F32)
    assert np.array_equal(C, (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float64))


# ------------------------------------------------- exact rational brute force

def _exact(Ad, Bd):
    M, K = Ad.shape
    N = Bd.shape[1]
    C = [[sum((Fraction(Ad[i, k]) * Fraction(Bd[k, j]) for k in range(K)), Fraction(0))
          for j in range(N)] for i in range(M)]
    S = [[sum((abs(Fraction(Ad[i, k]) * Fraction(Bd[k, j])) for k in range(K)), Fraction(0))
          for j in range(N)] for i in range(M)]
    return C, S


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [4, 16])
@pytest.mark.parametrize("dist", ["uniform", "normal"])
def test_bruteforce_exact_rationals(dt, n, dist):
    A, B = inputs.pair(n, n, n, dt, dist, seed=100 + n)
    Ad, Bd = A.double().numpy(), B.double().numpy()   # torch's decode, exact
    C, S = oracle.gemm(bits(A), bits(B), DT[dt])
    Cx, Sx = _exact(Ad, Bd)
    bound = n * 2.0 ** -53
    for i in range(n):
        for j in range(n):
            s = float(Sx[i][j])
            assert abs(Fraction(C[i, j]) - Cx[i][j]) <= Fraction(bound) * Sx[i][j], (i, j)
            assert abs(Fraction(S[i, j]) - Sx[i][j]) <= Fraction(bound) * Sx[i][j], (i, j)
            assert s > 0


# ------------------------------------------- layout, entries and arguments

@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_leading_dimensions_and_row_subsets(dt):
    M, N, K = 45, 38, 70
    A, B = inputs.pair(M, N, K, dt, "normal", seed=3)
    C, S = oracle.gemm(bits(A), bits(B), DT[dt])
    # padded rows (NaN in the padding) must not change anything
    Ap = inputs.with_ld(A, K + 9)
    Bp = inputs.with_ld(B, N + 5)
    C2, S2 = oracle.gemm(bits(Ap), bits(Bp), DT[dt])
    assert np.array_equal(C, C2) and np.array_equal(S, S2)
    # a block of rows of A gives that block of rows of C
    C3, _ = oracle.gemm(bits(A[10:20]), bits(B), DT[dt])
    assert np.array_equal(C3, C[10:20])


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_entries_equal_full_product(dt):
    M, N, K = 50, 61, 77
    A, B = inputs.pair(M, N, K, dt, "uniform", seed=4)
    C, S = oracle.gemm(bits(A), bits(B), DT[dt])
    rng = np.random.default_rng(0)
    rows = rng.integers(0, M, 200)
    cols = rng.integers(0, N, 200)
    Ce, Se = oracle.gemm_entries(bits(A), bits(B), DT[dt], rows, cols)
    assert np.array_equal(Ce, C[rows, cols]) and np.array_equal(Se, S[rows, cols])


def test_thread_count_does_not_change_result():
    A, B = inputs.pair(70, 90, 110, "bf16", "normal", seed=12)
    C1, S1 = oracle.gemm(bits(A), bits(B), oracle.BF16, nthreads=1)
    C8, S8 = oracle.gemm(bits(A), bits(B), oracle.BF16, nthreads=8)
    assert np.array_equal(C1, C8) and np.array_equal(S1, S8)


def test_bad_arguments_raise():
    A = np.zeros((3, 4), np.float32)
    B = np.zeros((5, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.gemm(A, B, oracle.F32)
    with pytest.raises(TypeError):
        oracle.gemm(A, np.zeros((4, 2), np.float64), oracle.F32)
    with pytest.raises(ValueError):
        oracle.gemm_entries(A, np.zeros((4, 2), np.float32), oracle.F32, [3], [0])


def test_empty_shapes():
    C, S = oracle.gemm(np.zeros((0, 5), np.float32), np.zeros((5, 3), np.float32), oracle.F32)
    assert C.shape == (0, 3)
    C, S = oracle.gemm(np.zeros((4, 0), np.uint16), np.zeros((0, 3), np.uint16), oracle.F16)
    assert C.shape == (4, 3) and np.all(C == 0) and np.all(S == 0)


# --------------------------------------------------------- comparison rule

def test_compare_rule_catches_planted_errors():
    rng = np.random.default_rng(1)
    want = rng.standard_normal((20, 30))
    S = np.abs(want) + 1.0
    ok = compare(want.astype(np.float32), want, S, tol=TOL_F32)
    assert ok.ok
    got = want.copy()
    got[7, 11] += 2 * TOL_F32 * S[7, 11]
    r = compare(got, want, S, tol=TOL_F32)
    assert not r.ok and r.first[:2] == (7, 11) and r.n_bad == 1
    got = want.copy()
    got[3, 4] += 0.5 * TOL_HALF * S[3, 4]
    assert compare(got, want, S, tol=TOL_HALF).ok
    got[3, 4] = np.nan
    assert not compare(got, want, S, tol=TOL_HALF).ok
    # exact mode: any difference fails, signed zeros are equal
    ints = np.round(want * 10)
    assert compare(ints.astype(np.float32), ints, S, exact=True).ok
    z = np.zeros((2, 2))
    assert compare(-z, z, z, exact=True).ok
    bumped = ints.copy()
    bumped[0, 0] += 1
    assert not compare(bumped, ints, S, exact=True).ok
    # where S == 0 equality is required even in tolerance mode
    zero_scale = np.zeros((1, 1))
    assert not compare(np.array([[1e-30]]), np.zeros((1, 1)), zero_scale, tol=TOL_F32).ok


# ---------------------------------------------------------------- output rounding and scaled update

def _finite_patterns(code):
    allbits = np.arange(65536, dtype=np.uint16)
    return allbits[np.isfinite(oracle.decode(allbits, code))]


@pytest.mark.parametrize("code", [oracle.F16, oracle.BF16])
def test_encode_roundtrip_exhaustive(code):
    """Every finite stored value (signed zeros and subnormals included) encodes back
    to its own bits."""
    pats = _finite_patterns(code)
    assert np.array_equal(oracle.encode(oracle.decode(pats, code), code), pats)


def test_encode_f32_roundtrip_sample():
    g = np.random.default_rng(7)
    w = g.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    w = np.concatenate([w, np.array([0, 0x80000000, 1, 0x807fffff, 0x7f7fffff, 0x00800000],
                                    dtype=np.uint32)])
    x = w.view(np.float32)
    w = w[np.isfinite(x)]
    got = oracle.encode(w.view(np.float32).astype(np.float64), oracle.F32).view(np.uint32)
    assert np.array_equal(got, w)


@pytest.mark.parametrize("code", [oracle.F16, oracle.BF16])
def test_encode_ties_to_even_exhaustive(code):
    """The midpoint of every pair of adjacent finite values goes to the one whose
    last significand bit is 0; a hair either side goes to the nearer one."""
    pats = _finite_patterns(code)
    pos = np.sort(pats[(pats & 0x8000) == 0])               # +0 .. max, increasing bits
    lo, hi = pos[:-1], pos[1:]
    a, b = oracle.decode(lo, code), oracle.decode(hi, code)
    mid = (a + b) / 2                                        # exact in binary64
    even = np.where((lo & 1) == 0, lo, hi)
    assert np.array_equal(oracle.encode(mid, code), even)
    assert np.array_equal(oracle.encode(-mid, code), even | 0x8000)
    gap = b - a
    assert np.array_equal(oracle.encode(mid - gap / 64, code), lo)
    assert np.array_equal(oracle.encode(mid + gap / 64, code), hi)


def test_encode_overflow_thresholds():
    # binary16: largest finite 65504, quantum 32 there: 65520 is the tie with 2^16 -> inf
    assert oracle.encode([65519.99, 65520.0, -65520.0, 1e30], oracle.F16).tolist() == \
        [0x7BFF, 0x7C00, 0xFC00, 0x7C00]
    # bfloat16: largest finite (2 - 2^-7) 2^127, quantum 2^120: the tie with 2^128 -> inf
    mx = (2 - 2 ** -7) * 2.0 ** 127
    assert oracle.encode([mx, mx + 2.0 ** 119, mx + 2.0 ** 119 * 0.999], oracle.BF16).tolist() == \
        [0x7F7F, 0x7F80, 0x7F7F]
    assert oracle.encode([float("nan")], oracle.F16)[0] & 0x7C00 == 0x7C00


def test_encode_matches_library_conversions():
    """Single roundings done by independent implementations: numpy's binary64 ->
    binary16 and binary64 -> binary32 casts, and torch's binary32 -> bfloat16 cast
    (its input exact in binary64, so one rounding)."""
    g = np.random.default_rng(11)
    x = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-9, 5, 20000),
                        g.uniform(-7e4, 7e4, 2000)])
    with np.errstate(over="ignore"):                          # overflow to inf is intended
        want16 = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.encode(x, oracle.F16), want16)
    assert np.array_equal(oracle.encode(x, oracle.F32), x.astype(np.float32))
    f = (g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000)).astype(np.float32)
    wantbf = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode(f.astype(np.float64), oracle.BF16), wantbf)


def test_epilogue_identity_and_unread_previous():
    acc = np.array([1.5, -2.25, 0.0, 3e-30])
    S = np.abs(acc) * 2
    out, sc = oracle.epilogue(acc, S, 1.0, 0.0, oracle.F32)
    assert np.array_equal(out, acc) and np.array_equal(sc, S)
    # beta == 0: the previous C is never read, NaN or not
    nan = np.full(acc.shape, np.nan, dtype=np.float32)
    out, _ = oracle.epilogue(acc, S, 2.0, 0.0, oracle.F32, nan)
    assert np.array_equal(out, 2 * acc)


@pytest.mark.parametrize("code", [oracle.F32, oracle.F16, oracle.BF16])
def test_epilogue_integers_exact(code):
    """alpha = 3, beta = -2 on integer products and an integer previous C: the update
    is exact integer arithmetic, and so is its scale."""
    g = np.random.default_rng(5)
    a = g.integers(-4, 5, (6, 9))
    b = g.integers(-4, 5, (9, 7))
    old = g.integers(-20, 21, (6, 7))
    tdt = {oracle.F32: torch.float32, oracle.F16: torch.float16, oracle.BF16: torch.bfloat16}[code]
    A, B = torch.from_numpy(a).to(tdt), torch.from_numpy(b).to(tdt)
    acc, S = oracle.gemm(bits(A), bits(B), code)
    old_bits = bits(torch.from_numpy(old).to(tdt))
    out, sc = oracle.epilogue(acc, S, 3.0, -2.0, code, old_bits)
    assert np.array_equal(out, (3 * (a @ b) - 2 * old).astype(float))
    assert np.array_equal(sc, (3 * (np.abs(a) @ np.abs(b)) + 2 * np.abs(old)).astype(float))


def test_epilogue_against_exact_rationals():
    """Powers-of-two alpha and beta make both products exact, so the one binary64
    addition is the only rounding: within half an ulp of the exact rational."""
    g = np.random.default_rng(9)
    acc = g.standard_normal(500)
    old = g.standard_normal(500).astype(np.float32)
    out, _ = oracle.epilogue(acc, np.abs(acc), 0.25, -8.0, oracle.F32, old)
    for x, y, o in zip(acc, old, out):
        exact = Fraction(0.25) * Fraction(float(x)) + Fraction(-8) * Fraction(float(y))
        assert abs(Fraction(float(o)) - exact) <= abs(exact) * Fraction(1, 2 ** 53)


def test_compare_output_rounding_term():
    want = np.array([1000.3, -2.0 ** -20, 0.0])
    got16 = oracle.decode(oracle.encode(want, oracle.F16), oracle.F16)
    scale = np.abs(want) * 1e-6           # a product whose own error budget is tiny
    assert compare(got16, want, scale, TOL_HALF, out_dtype=oracle.F16).ok
    # without the output term the rounded values do not pass
    assert not compare(got16, want, scale, TOL_HALF).ok
    # off by a whole unit of the output format: fails
    bad = got16.copy()
    bad[0] += 0.5
    assert not compare(bad, want, scale, TOL_HALF, out_dtype=oracle.F16).ok


# ---------------------------------------------------------------- INT8

def test_decode_i8_all_patterns_matches_numpy():
    allb = np.arange(256, dtype=np.uint8)
    assert np.array_equal(oracle.decode(allb, oracle.I8), allb.view(np.int8).astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(7, 9, 13), (64, 48, 300), (33, 70, 2048)])
def test_i8_product_exact_against_numpy_int64(M, N, K):
    """numpy's int64 matmul is exact; the oracle's binary64 sums of int8 products
    are exact too (every partial sum is an integer below 2^31)."""
    g = np.random.default_rng(M + N + K)
    A = g.integers(-128, 128, (M, K), dtype=np.int64).astype(np.int8)
    B = g.integers(-128, 128, (K, N), dtype=np.int64).astype(np.int8)
    C, S = oracle.gemm(A, B, oracle.I8)
    assert np.array_equal(C, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64))
    assert np.array_equal(S, (np.abs(A.astype(np.int64)) @ np.abs(B.astype(np.int64))).astype(np.float64))


def test_i8_extremes_exact():
    """-128 * -128 summed 2^17 times is 2^31: still exact in binary64."""
    K = 1 << 17
    A = np.full((1, K), -128, dtype=np.int8)
    B = np.full((K, 2), -128, dtype=np.int8)
    B[:, 1] = 127
    C, _ = oracle.gemm(A, B, oracle.I8)
    assert C[0, 0] == 2.0 ** 31 and C[0, 1] == -128 * 127 * K
