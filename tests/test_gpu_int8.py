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
           a_off=0, b_off=0, c_off=0, ws=False):
    """C = A x B (int8 CPU tensors, the product's operands; stored transposed on the
    GPU with ta / tb) through migemm_gemm_ex_variant with INT32 C inside a
    sentinel-filled buffer, or through migemm_gemm_ws lending the workspace
    migemm_workspace_size asks for (ws=True).  Returns (C as int64 numpy,
    whether padding is intact)."""
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
    pa = dAv.data_ptr() if K and M else None
    pb = dBv.data_ptr() if K and N else None
    stream = torch.cuda.current_stream().cuda_stream
    if ws:
        st, n = mg.migemm_workspace_size(variant, config, int(ta), int(tb), M, N, K, mg.I8, pa,
                                         lda, pb, ldb)
        assert st == mg.OK
        wt = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
        st = mg.migemm_gemm_ws(variant, config, int(ta), int(tb), M, N, K, mg.I8, pa, lda, pb,
                               ldb, 1.0, 0.0, mg.I32, dC.data_ptr(), ldc,
                               wt.data_ptr() if n else None, n, stream)
    else:
        st = mg.migemm_gemm_ex_variant(variant, config, int(ta), int(tb), M, N, K, mg.I8, pa,
                                       lda, pb, ldb, 1.0, 0.0, mg.I32, dC.data_ptr(), ldc,
                                       stream)
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


def _packed_case(M, N, K, ta=False, tb=False, lda=None, ldb=None, a_off=0, b_off=0, config=-1):
    A, B = inputs.pair(M, N, K, "i8", "uniform", seed=M + 5 * N + 7 * K + ta + 2 * tb)
    want = _want(A, B)
    v = -1 if config == -1 else mg.MFMA_I8
    say(f"i8 packed {_name(ta, tb)} {M}x{N}x{K} lda={lda} ldb={ldb} off={a_off},{b_off} "
        f"cfg={config}")
    C, intact = run_i8(A, B, v, config, ta=ta, tb=tb, lda=lda, ldb=ldb, a_off=a_off, b_off=b_off,
                       ws=True)
    assert intact
    bad = np.flatnonzero(C != want)
    assert bad.size == 0, f"{bad.size} differ; first {np.unravel_index(bad[0], C.shape)}"


def test_packed_selected_for_unaligned_operands():
    """Operands the direct kernels cannot read (K not a multiple of 16, rows off
    16-byte boundaries) with a workspace lent: the selection copies them into
    aligned zero-padded images (configuration 5) and runs the product of the
    copies, bit-exact: 1000^3 (then the 64x64 tile), 3000 x 3000 x 3072 with
    ldb = 3000 (A read in place, B copied; then the whole shape on the
    interleaved direct kernel), 4096 x 4096 x 4008 (both copied to K = 4096,
    then the ping-pong kernel)."""
    for (M, N, K, lda, ldb) in [(1000, 1000, 1000, 1000, 1000), (3000, 3000, 3072, 3072, 3000),
                                (4096, 4096, 4008, 4016, 4096)]:
        st, text = mg.migemm_describe_ex(-1, -1, 0, 0, M, N, K, mg.I8, None, lda, None, ldb,
                                         mg.I32, N, 1 << 40)
        assert st == mg.OK and mg._parse_description(text)["config"] == 5, text
        _packed_case(M, N, K, lda=lda, ldb=ldb)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_packed_every_layout_exact(ta, tb):
    """Configuration 5 asked for, every layout: K from 1 to past a k-tile, odd
    leading dimensions and element offsets of 1 and 3 (every source row off its
    16-byte boundary), ragged M and N."""
    for (M, N, K, pad, off) in [(300, 257, 77, 3, 1), (600, 520, 1000, 5, 3), (64, 65, 1, 0, 0),
                                (257, 300, 129, 9, 1), (512, 512, 256, 0, 0)]:
        lda = (M if ta else K) + pad
        ldb = (K if tb else N) + pad
        _packed_case(M, N, K, ta, tb, lda, ldb, off, off, config=5)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_interleaved_direct_exact(ta, tb):
    """Configuration 6, the direct 256x256 kernel with the interleaved schedule:
    ragged M and N (clamped loads, guarded stores), K a multiple of 16 but not of
    the 128-deep k-tile (a partial first k-tile), K = 16, padded leading
    dimensions in whole 16-byte chunks; bit-exact."""
    for (M, N, K, pad) in [(300, 264, 256, 0), (513, 640, 400, 16), (264, 296, 16, 0),
                           (1000, 1000, 1008, 32), (256, 512, 384, 0)]:
        A, B = inputs.pair(M, N, K, "i8", "uniform", seed=M + 2 * N + 5 * K + 7 * ta + 11 * tb)
        want = _want(A, B)
        lda = ((M if ta else K) + 15) // 16 * 16 + pad
        ldb = ((K if tb else N) + 15) // 16 * 16 + pad
        say(f"i8 interleaved {_name(ta, tb)} {M}x{N}x{K} lda={lda} ldb={ldb}")
        C, intact = run_i8(A, B, mg.MFMA_I8, 6, ta=ta, tb=tb, lda=lda, ldb=ldb)
        assert intact
        bad = np.flatnonzero(C != want)
        assert bad.size == 0, f"{bad.size} differ; first {np.unravel_index(bad[0], C.shape)}"


def test_interleaved_direct_extreme_sums():
    """Configuration 6 with K = 2^17 - 16 (a partial first k-tile of 112):
    (-128)(-128) summed 131056 times, exact."""
    M = N = 256
    K = (1 << 17) - 16
    A = torch.full((M, K), -128, dtype=torch.int8)
    A[M // 2:] = 127
    B = torch.full((K, N), -128, dtype=torch.int8)
    B[:, N // 2:] = 127
    want = np.empty((M, N), dtype=np.int64)
    want[:M // 2, :N // 2] = 16384 * K
    want[:M // 2, N // 2:] = -128 * 127 * K
    want[M // 2:, :N // 2] = -128 * 127 * K
    want[M // 2:, N // 2:] = 127 * 127 * K
    say("i8 interleaved extremes K=131056")
    C, intact = run_i8(A, B, mg.MFMA_I8, 6)
    assert intact and np.array_equal(C, want)


@pytest.mark.parametrize("block", range(4))
def test_random_cases_exact(block):
    """Seeded random INT8 cases: sizes biased to multiples of 16, 128 and 256 and
    one either side, every layout, padded leading dimensions and byte offsets
    (0, 1, 3, 16), through the selection with or without a workspace or on one
    configuration picked at random; bit-exact, padding of C untouched."""
    rng = np.random.default_rng(7700 + block)

    def dim(hi):
        u = rng.random()
        if u < 0.4:
            return 16 * int(rng.integers(1, hi // 16 + 1))
        if u < 0.7:
            m = int(rng.choice([16, 128, 256]))
            return int(min(hi, max(1, m * int(rng.integers(1, max(2, hi // m))) +
                                   int(rng.integers(-1, 2)))))
        return int(rng.integers(1, hi + 1))

    for i in range(25):
        M, N, K = dim(900), dim(900), dim(1400)
        ta, tb = bool(rng.random() < 0.3), bool(rng.random() < 0.3)
        pad = lambda: int(rng.choice([0, 0, 0, 16, 1, 3, 9]))
        lda, ldb = (M if ta else K) + pad(), (K if tb else N) + pad()
        off = int(rng.choice([0, 0, 0, 1, 3, 16]))
        route = str(rng.choice(["auto", "auto_ws", "config"]))
        v, c = -1, -1
        if route == "config":
            v, c = mg.MFMA_I8, int(rng.integers(0, mg.migemm_config_count(mg.MFMA_I8)))
        A, B = inputs.pair(M, N, K, "i8", "uniform", seed=100 * block + i)
        want = _want(A, B)
        say(f"i8 random block {block} case {i}: {_name(ta, tb)} {M}x{N}x{K} lda={lda} "
            f"ldb={ldb} off={off} {route} cfg={c}")
        C, intact = run_i8(A, B, v, c, ta=ta, tb=tb, lda=lda, ldb=ldb, a_off=off, b_off=off,
                           ws=route != "auto")
        assert intact
        bad = np.flatnonzero(C != want)
        assert bad.size == 0, f"{bad.size} differ; first {np.unravel_index(bad[0], C.shape)}"


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_split_k_exact(ta, tb):
    """Configuration 7: slices of K (whole 128-deep k-tiles, the last the rest) on
    the interleaved direct kernel, their INT32 sums added by the integer sum
    kernel; ragged M and N (whole 16-byte chunks where they are a contiguous
    side), K a multiple of 16 only (the last slice starts with a partial
    k-tile), every layout, and with both operands k-contiguous an M x N that is
    not a multiple of 4; bit-exact."""
    cases = [(256, 256, 8192), (304, 272, 4112), (272, 144, 2064), (64, 64, 16384)]
    if not ta and tb:
        cases.append((257, 129, 2064))
    for (M, N, K) in cases:
        A, B = inputs.pair(M, N, K, "i8", "uniform", seed=M + 3 * N + 5 * K + 7 * ta + 11 * tb)
        want = _want(A, B)
        lda = ((M if ta else K) + 15) // 16 * 16
        ldb = ((K if tb else N) + 15) // 16 * 16
        st, text = mg.migemm_describe_ex(mg.MFMA_I8, 7, int(ta), int(tb), M, N, K, mg.I8, None,
                                         lda, None, ldb, mg.I32, N, 1 << 40)
        assert st == mg.OK and mg._parse_description(text)["launches"] == 2, text
        say(f"i8 split-K {_name(ta, tb)} {M}x{N}x{K} lda={lda} ldb={ldb}")
        C, intact = run_i8(A, B, mg.MFMA_I8, 7, ta=ta, tb=tb, lda=lda, ldb=ldb, ws=True)
        assert intact
        bad = np.flatnonzero(C != want)
        assert bad.size == 0, f"{bad.size} differ; first {np.unravel_index(bad[0], C.shape)}"


def test_split_k_selected_and_extreme():
    """The selection's split-K on 1024 x 1024 x 8192, and the extreme sums at the
    K limit split over 16 slices (each slice sum and the total exact)."""
    A, B = inputs.pair(1024, 1024, 8192, "i8", "uniform", seed=77)
    st, text = mg.migemm_describe_ex(-1, -1, 0, 0, 1024, 1024, 8192, mg.I8, None, 8192, None,
                                     1024, mg.I32, 1024, 1 << 40)
    assert st == mg.OK and mg._parse_description(text)["config"] == 7, text
    say("i8 split-K 1024x1024x8192 through the selection")
    C, intact = run_i8(A, B, ws=True)
    assert intact and np.array_equal(C, _want(A, B))
    K = (1 << 17) - 16
    A = torch.full((32, K), -128, dtype=torch.int8)
    A[16:] = 127
    B = torch.full((K, 32), -128, dtype=torch.int8)
    B[:, 16:] = 127
    want = np.empty((32, 32), dtype=np.int64)
    want[:16, :16] = 16384 * K
    want[:16, 16:] = -128 * 127 * K
    want[16:, :16] = -128 * 127 * K
    want[16:, 16:] = 127 * 127 * K
    say("i8 split-K extremes K=131056")
    C, intact = run_i8(A, B, mg.MFMA_I8, 7, ws=True)
    assert intact and np.array_equal(C, want)
