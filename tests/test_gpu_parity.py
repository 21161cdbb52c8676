"""GPU parity: every variant and configuration against the CPU oracle, through the C ABI.

Bar: bit-exact where every partial sum is an integer below 2^24 (small-integer
inputs, all-ones, identity, permutation); otherwise |C - C_ref| <= tol * S per
element with S = sum_k |A[i][k] B[k][j]|, tol = 1e-4 (FP32) or 5e-4
(FP16/BF16 with FP32 accumulation).  Inputs are seeded; C is poisoned with NaN
before each call so an unwritten element fails.
"""
import numpy as np
import pytest
import torch

import dense_gemm_16_amd as mg
from dense_gemm_16_amd import inputs
from gpu_helpers import check, run_gemm, say

pytestmark = pytest.mark.gpu

# (variant, config) pairs per dtype: every configuration of every variant.
def _cases(dtype):
    code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    out = []
    for v in range(mg.migemm_variant_count()):
        if mg.migemm_variant_supports(v, code):
            out += [(v, c) for c in range(mg.migemm_config_count(v))]
    return out


SHAPES = [(1, 1, 1), (17, 33, 9), (64, 64, 64), (130, 70, 200), (300, 257, 129),
          (512, 512, 512), (600, 520, 300)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_every_config_matches_oracle(dtype):
    for (M, N, K) in SHAPES:
        A, B = inputs.pair(M, N, K, dtype, "uniform", seed=M * 7 + N * 3 + K)
        ref = None
        for v, c in _cases(dtype):
            if v == mg.NAIVE and M * N * K > 64 * 1024 * 1024:
                continue
            say(f"every_config {dtype} {M}x{N}x{K} variant={mg.migemm_variant_name(v)} cfg={c}")
            C, _ = run_gemm(A, B, dtype, variant=v, config=c)
            from gpu_helpers import oracle_ref
            ref = ref or oracle_ref(A, B, dtype)
            check(C, A, B, dtype, ref=ref)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_small_integers_bit_exact_every_config(dtype):
    M, N, K = 200, 136, 1000
    A, B = inputs.pair(M, N, K, dtype, "int", seed=5)
    ref = None
    for v, c in _cases(dtype):
        say(f"int_exact {dtype} variant={mg.migemm_variant_name(v)} cfg={c}")
        C, _ = run_gemm(A, B, dtype, variant=v, config=c)
        from gpu_helpers import oracle_ref
        ref = ref or oracle_ref(A, B, dtype)
        check(C, A, B, dtype, exact=True, ref=ref)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_structured_cases_exact(dtype):
    t = inputs.TORCH_DTYPES[dtype]
    n, p = 96, 80
    B = inputs.draw((n, p), dtype, "int", torch.Generator().manual_seed(1))
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(2))
    P = torch.zeros(n, n)
    P[torch.arange(n), perm] = 1.0
    I = torch.eye(n)
    for v, c in _cases(dtype):
        say(f"structured {dtype} variant={mg.migemm_variant_name(v)} cfg={c}")
        C, _ = run_gemm(I.to(t), B, dtype, variant=v, config=c)
        assert torch.equal(C, B.float()), "identity"
        C, _ = run_gemm(P.to(t), B, dtype, variant=v, config=c)
        assert torch.equal(C, B.float()[perm]), "permutation"
        ones_a, ones_b = torch.ones(33, 777).to(t), torch.ones(777, 65).to(t)
        C, _ = run_gemm(ones_a, ones_b, dtype, variant=v, config=c)
        assert torch.all(C == 777), "all-ones"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_edge_sweep_selected_path(dtype):
    dims = [1, 15, 16, 17, 63, 65, 127, 129, 255, 257]
    rng = np.random.default_rng(3)
    for trial in range(24):
        M, N, K = (int(x) for x in rng.choice(dims, 3))
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=trial)
        say(f"edge_sweep {dtype} {M}x{N}x{K}")
        C, _ = run_gemm(A, B, dtype)
        check(C, A, B, dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_leading_dims_misalignment_and_poison(dtype):
    M, N, K = 197, 211, 233
    A, B = inputs.pair(M, N, K, dtype, "uniform", seed=9)
    for v, c in _cases(dtype):
        if v == mg.NAIVE:
            continue
        for (lda, ldb, ldc, ao, bo, co) in [(K + 1, N + 3, N + 1, 0, 0, 0),
                                            (K + 8, N + 8, N + 4, 1, 1, 1),
                                            (K, N, N, 3, 5, 2)]:
            say(f"ld {dtype} variant={mg.migemm_variant_name(v)} cfg={c} "
                f"ld=({lda},{ldb},{ldc}) off=({ao},{bo},{co})")
            C, cbuf = run_gemm(A, B, dtype, variant=v, config=c, lda=lda, ldb=ldb, ldc=ldc,
                               a_off=ao, b_off=bo, c_off=co)
            check(C, A, B, dtype)
            # everything outside the M x N window is still the NaN poison
            full = cbuf.cpu()
            inside = torch.zeros_like(full, dtype=torch.bool)
            for r in range(M):
                inside[co + r * ldc: co + r * ldc + N] = True
            assert torch.all(torch.isnan(full[~inside])), "wrote outside the C window"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_degenerate_shapes(dtype):
    # K == 0 writes zeros; M == 0 / N == 0 are no-ops
    A = torch.zeros(37, 0).to(inputs.TORCH_DTYPES[dtype])
    B = torch.zeros(0, 41).to(inputs.TORCH_DTYPES[dtype])
    for v, c in _cases(dtype):
        say(f"degenerate K=0 {dtype} variant={v} cfg={c}")
        C, _ = run_gemm(A, B, dtype, variant=v, config=c)
        assert torch.all(C == 0)
    C, _ = run_gemm(torch.zeros(0, 5).to(A.dtype), torch.zeros(5, 3).to(A.dtype), dtype)
    assert C.shape == (0, 3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_k_trip_counts(dtype):
    # 1..5 k-tiles plus a tail: exercises the double-buffer hand-off; tails of
    # whole 16-byte chunks take the direct kernel's zero-filled last k-tile,
    # others the register-staged kernel
    bk = 32 if dtype == "f32" else 64
    chunk = 4 if dtype == "f32" else 8
    for kt in range(1, 6):
        for tail in (0, 1, chunk, bk - chunk, bk - 1):
            K = kt * bk + tail
            A, B = inputs.pair(256, 256, K, dtype, "int", seed=K)
            say(f"k_trips {dtype} K={K}")
            C, _ = run_gemm(A, B, dtype)
            check(C, A, B, dtype, exact=True)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_run_to_run_bitwise_determinism(dtype):
    A, B = inputs.pair(700, 600, 900, dtype, "normal", seed=17)
    for v, c in _cases(dtype):
        if v == mg.NAIVE:
            continue
        say(f"determinism {dtype} variant={v} cfg={c}")
        C1, _ = run_gemm(A, B, dtype, variant=v, config=c)
        C2, _ = run_gemm(A, B, dtype, variant=v, config=c)
        assert torch.equal(C1, C2)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_direct_staging_edges(dtype):
    """Configurations with direct global->LDS staging: ragged M, N a multiple of 8
    that is not a multiple of the tile, K a multiple of 64, padded leading
    dimensions (multiples of 8), and a K of one k-tile."""
    names = [mg.migemm_config_name(mg.MFMA16, c) for c in range(mg.migemm_config_count(mg.MFMA16))]
    direct = [c for c, n in enumerate(names) if n.startswith("direct")]
    assert direct
    shapes = [(300, 264, 128, None, None), (1000, 520, 640, None, None), (256, 256, 64, None, None),
              (37, 8, 192, None, None), (513, 776, 256, 264, 784), (64, 1024, 1024, 1032, 1040)]
    for (M, N, K, lda, ldb) in shapes:
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=M + N + K)
        ref = None
        for c in direct:
            say(f"direct {dtype} {M}x{N}x{K} lda={lda} ldb={ldb} cfg={names[c]}")
            C, _ = run_gemm(A, B, dtype, variant=mg.MFMA16, config=c, lda=lda, ldb=ldb)
            from gpu_helpers import oracle_ref
            ref = ref or oracle_ref(A, B, dtype)
            check(C, A, B, dtype, ref=ref)


RAGGED_K_SHAPES = [(300, 264, 72, None, None), (1000, 520, 200, None, None),
                   (256, 256, 8, None, None), (37, 8, 1096, None, None),
                   (513, 776, 136, 144, 784), (129, 128, 1000, None, None),
                   (2048, 64, 2056, None, None)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_direct_ragged_k(dtype):
    """Direct-staged configurations that zero-fill a partial k-tile (the last one;
    the first one for the 256x256 interleaved configuration 10): K a multiple of
    the 16-byte chunk (8 elements, 4 for FP32) but not of the k-tile, from one
    chunk (K = 8) to many k-tiles, with ragged M and N and padded leading
    dimensions.  Every direct configuration runs each shape (those without a
    partial k-tile take the register-staged kernel)."""
    v = mg.REGTILE_MFMA if dtype == "f32" else mg.MFMA16
    names = [mg.migemm_config_name(v, c) for c in range(mg.migemm_config_count(v))]
    direct = [c for c, n in enumerate(names) if n.startswith("direct")]
    assert direct
    for (M, N, K, lda, ldb) in RAGGED_K_SHAPES:
        if dtype == "f32":
            K = K // 2  # still a multiple of 4, not of 32
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=3 * M + N + K)
        ref = None
        for c in direct:
            say(f"ragged_k {dtype} {M}x{N}x{K} lda={lda} ldb={ldb} cfg={names[c]}")
            C, _ = run_gemm(A, B, dtype, variant=v, config=c, lda=lda, ldb=ldb)
            from gpu_helpers import oracle_ref
            ref = ref or oracle_ref(A, B, dtype)
            check(C, A, B, dtype, ref=ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_direct_ragged_k_layouts_and_general_output(dtype):
    """The partial k-tile in every operand layout (row images and k-row images
    both end inside it; for configuration 10 both start inside its first
    k-tile), with the general output step into a 16-bit C and small integers
    compared bit for bit."""
    from gpu_helpers import check_ex, oracle_ref, padding_untouched, run_gemm_ex
    v = mg.REGTILE_MFMA if dtype == "f32" else mg.MFMA16
    cfgs = (8, 10) if dtype == "f32" else (7, 10, 13, 16)
    K = 100 if dtype == "f32" else 200
    M, N = 264, 136
    for kind in ("normal", "int"):
        A, B = inputs.pair(M, N, K, dtype, kind, seed=K + (kind == "int"))
        ref = oracle_ref(A, B, dtype)
        old = (torch.rand((M, N), generator=torch.Generator().manual_seed(7)) - 0.5).to(
            torch.bfloat16)
        for ta in (False, True):
            for tb in (False, True):
                for c in cfgs:
                    say(f"ragged_k layouts {dtype} {kind} ta={ta} tb={tb} cfg={c}")
                    C, buf, mask = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None, variant=v,
                                               config=c, ta=ta, tb=tb)
                    check_ex(C, A, B, dtype, 1.0, 0.0, 0, None, ref=ref, exact=kind == "int")
                    assert padding_untouched(buf, mask)
                    if kind == "normal":
                        C, buf, mask = run_gemm_ex(A, B, dtype, 0.5, -1.0, 2, old, variant=v,
                                                   config=c, ta=ta, tb=tb)
                        check_ex(C, A, B, dtype, 0.5, -1.0, 2, old, ref=ref)
                        assert padding_untouched(buf, mask)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_partial_first_k_tile_full_rounds(dtype):
    """The 256x256 interleaved configuration selected for a K that ends inside a
    k-tile: its first k-tile holds the K mod 64 leftover k (the rest of its LDS
    image zero-filled in the prologue) and every later k-tile is whole.  Full
    rounds of 256 workgroups, K from one chunk (a single, partial k-tile) to
    several k-tiles with every leftover 8 .. 56, ragged M and N (the split of
    the last bands runs after the whole tiles), compared with the oracle; small
    integers bit for bit."""
    from gpu_helpers import oracle_ref
    for (M, N, K, dist) in [(4096, 4096, 8, "normal"), (4096, 4096, 200, "normal"),
                            (4096, 4096, 136, "int"), (4100, 4104, 248, "normal"),
                            (4096, 4096, 120, "int"), (4096, 4096, 328, "normal")]:
        A, B = inputs.pair(M, N, K, dtype, dist, seed=M + N + K)
        st, v, c = mg.migemm_select(M, N, K, inputs.DTYPE_CODES[dtype], None, K, None, N,
                                    None, N)
        assert st == mg.OK and (v, c) == (mg.MFMA16, 10), (v, c)
        say(f"partial first k-tile {dtype} {M}x{N}x{K} {dist}")
        C, _ = run_gemm(A, B, dtype)
        check(C, A, B, dtype, exact=dist == "int", ref=oracle_ref(A, B, dtype))
