"""GPU parity for the configurations that need whole workgroup tiles (the
ping-pong 256x256 schedule), through the C ABI, against the CPU oracle.

Shapes are whole 256x256 tiles with 1, 2, 3 and more k-tiles of 64, with dense
and padded leading dimensions, in all four operand layouts and with the general
output step; a ragged shape checks that such a configuration hands other
shapes to its fallback.  Bar as in the other parity tests: tolerance
5e-4 * sum|A B| for 16-bit inputs, bit-exact on small integers.
"""
import pytest
import torch

import dense_gemm_16_amd as mg
from dense_gemm_16_amd import inputs
from gpu_helpers import check, check_ex, oracle_ref, run_gemm, run_gemm_ex, say

pytestmark = pytest.mark.gpu


def _whole_tile_configs():
    names = [mg.migemm_config_name(mg.MFMA16, c) for c in range(mg.migemm_config_count(mg.MFMA16))]
    out = [c for c, n in enumerate(names) if "pingpong" in n]
    assert out, "no whole-tile configuration in the table"
    return out


SHAPES = [(256, 256, 64, None, None), (256, 512, 128, None, None), (512, 256, 192, None, None),
          (768, 512, 1024, 1032, 520), (512, 768, 320, 328, 776)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_whole_tiles_match_oracle(dtype):
    for (M, N, K, lda, ldb) in SHAPES:
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=M + 3 * N + 7 * K)
        ref = oracle_ref(A, B, dtype)
        for c in _whole_tile_configs():
            say(f"whole_tiles {dtype} {M}x{N}x{K} lda={lda} ldb={ldb} cfg={c}")
            C, _ = run_gemm(A, B, dtype, variant=mg.MFMA16, config=c, lda=lda, ldb=ldb)
            check(C, A, B, dtype, ref=ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_whole_tiles_integers_exact(dtype):
    M, N, K = 512, 512, 640
    A, B = inputs.pair(M, N, K, dtype, "int", seed=31)
    ref = oracle_ref(A, B, dtype)
    for c in _whole_tile_configs():
        say(f"whole_tiles_int {dtype} cfg={c}")
        C, _ = run_gemm(A, B, dtype, variant=mg.MFMA16, config=c)
        check(C, A, B, dtype, exact=True, ref=ref)


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)])
def test_whole_tiles_transposed(ta, tb):
    dtype = "bf16"
    for (M, N, K) in [(256, 256, 64), (512, 768, 192)]:
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=M + N + K + 2 * ta + tb)
        ref = oracle_ref(A, B, dtype)
        for c in _whole_tile_configs():
            say(f"whole_tiles_layout {M}x{N}x{K} ta={ta} tb={tb} cfg={c}")
            C, _, _ = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, variant=mg.MFMA16, config=c,
                                  ta=ta, tb=tb)
            check_ex(C, A, B, dtype, 1.0, 0.0, 0, ref=ref)


@pytest.mark.parametrize("c_code", [0, 2])
def test_whole_tiles_general_update(c_code):
    dtype = "f16"
    M, N, K = 512, 512, 256
    A, B = inputs.pair(M, N, K, dtype, "uniform", seed=77)
    g = torch.Generator().manual_seed(78)
    tdt = {0: torch.float32, 2: torch.bfloat16}[c_code]
    c_old = (torch.rand(M, N, generator=g) * 2 - 1).to(tdt)
    ref = oracle_ref(A, B, dtype)
    for c in _whole_tile_configs():
        say(f"whole_tiles_general c={c_code} cfg={c}")
        C, _, _ = run_gemm_ex(A, B, dtype, 0.5, -1.0, c_code, c_old=c_old, variant=mg.MFMA16,
                              config=c)
        check_ex(C, A, B, dtype, 0.5, -1.0, c_code, c_old=c_old, ref=ref)


def test_ragged_shape_falls_back():
    """M or N not a whole number of tiles: the configuration runs its fallback
    kernel and the result still matches."""
    dtype = "bf16"
    for (M, N, K) in [(300, 256, 128), (256, 264, 128), (520, 1000, 192)]:
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=M * N + K)
        ref = oracle_ref(A, B, dtype)
        for c in _whole_tile_configs():
            say(f"whole_tiles_fallback {M}x{N}x{K} cfg={c}")
            C, _ = run_gemm(A, B, dtype, variant=mg.MFMA16, config=c)
            check(C, A, B, dtype, ref=ref)
