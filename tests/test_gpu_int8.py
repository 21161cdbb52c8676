"""INT8 inputs, exact INT32 sums (MIGEMM_MFMA_I8), bit-exact against the oracle.

Every configuration in every operand layout on ragged and aligned shapes, K
not a multiple of the 16-element chunk, the extreme sums at the K limit
(-128 * -128 summed 2^17 - 1 times, just below 2^31), padded and misaligned
storage with the padding of C untouched, and K == 0 (the 8192^3 shape is
compared in full in test_gpu_fullsize.py).
"""
import numpy as np
import pytest
import torch

import dense_gemm_16_amd as mg
import oracle
from dense_gemm_16_amd import inputs
from gpu_helpers import say

pytestmark = pytest.mark.gpu

SENTINEL = -2147483647
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _name(ta, tb):
    return ("T" if ta else "N") + ("T" if tb else "N")


def run_i8(A, B, variant=-1, config=-1, ta=False, tb=False, lda=None, ldb=None, ldc=None,
           a_off=0, b_off=0, c_off=0):
    """C = A x B (int8 CPU tensors, the product's operands; stored transposed on the
    GPU with ta / tb) through migemm_gemm_ex_variant with INT32 C inside a
    sentinel-filled buffer.  Returns (C as int64 numpy, whether padding is intact)."""
    M, K = A.shape
    N = B.shape[1]
    sA = A.t().contiguous() if ta else A
    sB = B.t().contiguous() if tb else B
    dA = torch.zeros((a_off + max(sA.shape[0], 1) * (lda or max(sA.shape[1], 1)) + 64,),
                     dtype=torch.int8, device="cuda")
    lda = lda or max(sA.shape[1], 1)
    ldb = ldb or max(sB.shape[1], 1)
    dAv = dA[a_off:a_off + sA.shape[0] * lda].view(sA.shape[0], lda)[:, :sA.shape[1]]
    dAv.copy_(sA.cuda())
    dB = torch.zeros((b_off + max(sB.shape[0], 1) * ldb + 64,), dtype=torch.int8, device="cuda")
    dBv = dB[b_off:b_off + sB.shape[0] * ldb].view(sB.shape[0], ldb)[:, :sB.shape[1]]
    dBv.copy_(sB.cuda())
    ldc = ldc or max(N, 1)
    cbuf = torch.full((c_off + max(M, 1) * ldc + 64,), SENTINEL, dtype=torch.int32, device="cuda")
    dC = cbuf[c_off:c_off + M * ldc].view(M, ldc)[:, :N]
    st = mg.migemm_gemm_ex_variant(variant, config, int(ta), int(tb), M, N, K, mg.I8,
                                   dAv.data_ptr() if K and M else None, lda,
                                   dBv.data_ptr() if K and N else None, ldb, 1.0, 0.0, mg.I32,
                                   dC.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mg.OK, mg.migemm_status_string(st)
    mask = torch.zeros(cbuf.shape, dtype=torch.bool)
    mask[c_off:c_off + M * ldc].view(M, ldc)[:, :N] = True
    intact = bool((cbuf.cpu()[~mask] == SENTINEL).all())
    return dC.cpu().numpy().astype(np.int64), intact


def _want(A, B):
    C, _ = oracle.gemm(A.numpy(), B.numpy(), oracle.I8)
    return C


def _configs():
    return [(-1, -1)] + [(mg.MFMA_I8, c) for c in range(mg.migemm_config_count(mg.MFMA_I8))]


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_every_config_exact(ta, tb):
    for (M, N, K) in [(1, 1, 1), (97, 130, 200), (264, 296, 256), (300, 257, 77), (513, 640, 384)]:
        A, B = inputs.pair(M, N, K, "i8", "uniform", seed=M + N + K + 3 * ta + 5 * tb)
        want = _want(A, B)
        for v, c in _configs():
            say(f"i8 {_name(ta, tb)} {M}x{N}x{K} variant={v} cfg={c}")
            C, intact = run_i8(A, B, v, c, ta=ta, tb=tb)
            assert intact
            bad = np.flatnonzero(C != want)
            assert bad.size == 0, f"{bad.size} differ; first {np.unravel_index(bad[0], C.shape)}"


WHOLE = [(256, 256, 128, None, None), (256, 512, 256, None, None), (512, 256, 384, None, None),
         (768, 512, 1024, 1056, 528), (512, 768, 640, 656, 784)]


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_whole_tiles_exact(ta, tb):
    """Whole 256 x 256 tiles with 1, 2, 3 and more 128-deep k-tiles, dense and
    padded leading dimensions (multiples of 16): the shapes the direct ping-pong
    configuration runs itself, in every layout, bit-exact."""
    direct = [c for c in range(mg.migemm_config_count(mg.MFMA_I8))
              if "pingpong" in mg.migemm_config_name(mg.MFMA_I8, c)]
    assert direct
    for (M, N, K, lda, ldb) in WHOLE:
        A, B = inputs.pair(M, N, K, "i8", "uniform", seed=M + 2 * N + 3 * K + 7 * ta + 11 * tb)
        want = _want(A, B)
        if ta and lda:
            lda = M + 32
        if tb and ldb:
            ldb = K + 16
        for c in [-1] + direct:
            v = -1 if c == -1 else mg.MFMA_I8
            say(f"i8 whole {_name(ta, tb)} {M}x{N}x{K} lda={lda} ldb={ldb} cfg={c}")
            C, intact = run_i8(A, B, v, c, ta=ta, tb=tb, lda=lda, ldb=ldb)
            assert intact
            bad = np.flatnonzero(C != want)
            assert bad.size == 0, f"{bad.size} differ; first {np.unravel_index(bad[0], C.shape)}"


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_ragged_bands_split_exact(ta, tb):
    """A partial last band of 256-row tiles or 256-column tiles: the whole tiles
    run on the direct ping-pong kernel, then the rows past them (up to 16 on the
    skinny kernel, 64-deep k-steps, k-rows transposed through LDS; more on the
    64x64 tile), then the columns past them (the transposed product on the
    skinny kernel when they are whole 16-byte chunks, else the 64x64 tile); a
    128x128-tile product one band past a round.  Selected automatically and with
    configurations 3 and 4 asked for; bit-exact."""
    cases = [(4100, 4096, 128), (4096, 4112, 128), (4100, 4112, 256), (4160, 4096, 128),
             (4096, 4104, 128), (2056, 2048, 128)]
    for (M, N, K) in cases:
        A, B = inputs.pair(M, N, K, "i8", "uniform", seed=M + 2 * N + 3 * K + 7 * ta + 11 * tb)
        want = _want(A, B)
        lda = ((M if ta else K) + 15) // 16 * 16
        ldb = ((K if tb else N) + 15) // 16 * 16
        for (v, c) in [(-1, -1), (mg.MFMA_I8, 3), (mg.MFMA_I8, 4)]:
            say(f"i8 split {_name(ta, tb)} {M}x{N}x{K} lda={lda} ldb={ldb} cfg={c}")
            C, intact = run_i8(A, B, v, c, ta=ta, tb=tb, lda=lda, ldb=ldb)
            assert intact
            bad = np.flatnonzero(C != want)
            assert bad.size == 0, f"{bad.size} differ; first {np.unravel_index(bad[0], C.shape)}"


def test_whole_tiles_extreme_sums():
    """The largest K the direct configuration takes itself (a multiple of 128
    below 2^17): (-128)(-128) summed 130944 times is 2^31 - 2^21, still exact."""
    M = N = 256
    K = (1 << 17) - 128
    A = torch.full((M, K), -128, dtype=torch.int8)
    A[M // 2:] = 127
    B = torch.full((K, N), -128, dtype=torch.int8)
    B[:, N // 2:] = 127
    want = np.empty((M, N), dtype=np.int64)
    want[:M // 2, :N // 2] = 16384 * K
    want[:M // 2, N // 2:] = -128 * 127 * K
    want[M // 2:, :N // 2] = -128 * 127 * K
    want[M // 2:, N // 2:] = 127 * 127 * K
    say("i8 whole-tile extremes K=130944")
    C, intact = run_i8(A, B)
    assert intact and np.array_equal(C, want)


def test_extreme_sums_at_the_k_limit():
    """K = 2^17 - 1: (-128)(-128) sums to 2^31 - 2^14 and (-128)(127) to its negative
    counterpart, the largest magnitudes an INT32 result can take here."""
    K = (1 << 17) - 1
    A = torch.full((16, K), -128, dtype=torch.int8)
    A[8:] = 127
    B = torch.full((K, 16), -128, dtype=torch.int8)
    B[:, 8:] = 127
    say("i8 extremes K=2^17-1")
    for v, c in _configs():
        C, _ = run_i8(A, B, v, c)
        want = np.empty((16, 16), dtype=np.int64)
        want[:8, :8] = 16384 * K
        want[:8, 8:] = -128 * 127 * K
        want[8:, :8] = -128 * 127 * K
        want[8:, 8:] = 127 * 127 * K
        assert np.array_equal(C, want)


@pytest.mark.parametrize("ta,tb", [(False, False), (True, True)])
def test_padded_and_misaligned(ta, tb):
    M, N, K = 200, 136, 320
    A, B = inputs.pair(M, N, K, "i8", "uniform", seed=31)
    want = _want(A, B)
    for off in (0, 1):
        for v, c in _configs():
            say(f"i8 padded {_name(ta, tb)} off={off} variant={v} cfg={c}")
            C, intact = run_i8(A, B, v, c, ta=ta, tb=tb, lda=(M if ta else K) + 32,
                               ldb=(K if tb else N) + 16, ldc=N + 7, a_off=off, b_off=off,
                               c_off=3)
            assert intact and np.array_equal(C, want)


def test_empty_k_writes_zeros():
    A = torch.zeros((5, 0), dtype=torch.int8)
    B = torch.zeros((0, 9), dtype=torch.int8)
    C, intact = run_i8(A, B, ldc=12)
    assert intact and np.all(C == 0)
