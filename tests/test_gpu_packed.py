"""The packed FP16/BF16 path (mfma16 configurations 11 and 12): A and B are
copied into zero-padded k-contiguous images in a workspace the caller lends
(migemm_gemm_ws) and the direct kernel multiplies those as A x B^T.

Checked against the oracle: K not a multiple of the 64-k tile (down to K = 1),
odd leading dimensions and operands that start off a 16-byte boundary (the
operand buffers are NaN-filled around each window, so a read outside an operand
shows up in C), all four storage layouts, the general output step, exact
integer inputs, the automatic selection for shapes that need packing, calls on
two streams each with its own workspace, and calls that lend no, too little or
a misaligned workspace (the product then runs in place).
"""
import pytest
import torch

import dense_gemm_16_amd as mg
from dense_gemm_16_amd import inputs
from gpu_helpers import (DT_CODE, check_ex, oracle_ref, padding_untouched, run_gemm_ex, say,
                         to_device_with_ld)

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]
PACKED = [11, 12]


def _name(ta, tb):
    return ("T" if ta else "N") + ("T" if tb else "N")


def test_packed_configs_named():
    for c in PACKED:
        assert mg.migemm_config_name(mg.MFMA16, c).startswith("packed")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_packed_ragged_k_every_layout(dtype, ta, tb):
    for (M, N, K) in [(1, 1, 1), (7, 9, 5), (130, 97, 65), (300, 264, 200), (257, 513, 130)]:
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=M + 2 * N + 3 * K + 5 * ta + 7 * tb)
        ref = oracle_ref(A, B, dtype)
        for c in PACKED:
            say(f"packed {_name(ta, tb)} {dtype} {M}x{N}x{K} cfg={c}")
            C, _, _ = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None, variant=mg.MFMA16, config=c,
                                  ta=ta, tb=tb)
            check_ex(C, A, B, dtype, 1.0, 0.0, 0, None, ref=ref)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_packed_odd_ld_and_misaligned(ta, tb):
    M, N, K = 203, 170, 301
    for dtype in ("f16", "bf16"):
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=31 + ta + 2 * tb)
        ref = oracle_ref(A, B, dtype)
        lda = (M if ta else K) + 3
        ldb = (K if tb else N) + 5
        for a_off, b_off in ((1, 3), (0, 1), (7, 0)):
            for c in PACKED:
                say(f"packed odd-ld {_name(ta, tb)} {dtype} offs={a_off},{b_off} cfg={c}")
                C, _, _ = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None, variant=mg.MFMA16,
                                      config=c, ta=ta, tb=tb, lda=lda, ldb=ldb, a_off=a_off,
                                      b_off=b_off)
                check_ex(C, A, B, dtype, 1.0, 0.0, 0, None, ref=ref)


def test_packed_transposing_copy_every_misalignment():
    """The transposing copy (row-major B, A given transposed) reads each k-row's
    64 elements as the 16-byte aligned chunks that cover them, so every start
    position within a chunk occurs: element offsets 0 to 7 of the operand against
    leading dimensions of every residue modulo 8, on shapes with ragged tiles in
    both directions and a K that ends inside a tile."""
    M, N, K = 130, 200, 150
    for (ta, tb) in ((False, False), (True, True)):
        A, B = inputs.pair(M, N, K, "bf16", "normal", seed=77 + ta)
        ref = oracle_ref(A, B, "bf16")
        for off in range(8):
            for pad in range(8):
                lda = (M if ta else K) + pad
                ldb = (K if tb else N) + (pad + off) % 8
                say(f"transposing copy {_name(ta, tb)} off={off} lda={lda} ldb={ldb}")
                C, _, _ = run_gemm_ex(A, B, "bf16", 1.0, 0.0, 0, None, variant=mg.MFMA16,
                                      config=12, ta=ta, tb=tb, lda=lda, ldb=ldb,
                                      a_off=(off + 3) % 8, b_off=off)
                check_ex(C, A, B, "bf16", 1.0, 0.0, 0, None, ref=ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_packed_general_output(dtype):
    M, N, K = 190, 321, 77
    A, B = inputs.pair(M, N, K, dtype, "normal", seed=8)
    ref = oracle_ref(A, B, dtype)
    for c_code in (0, 1, 2):
        old = (torch.rand((M, N), generator=torch.Generator().manual_seed(c_code)) - 0.5).to(
            {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[c_code])
        for ta, tb in LAYOUTS:
            for c in PACKED:
                say(f"packed general {_name(ta, tb)} {dtype} c_dtype={c_code} cfg={c}")
                C, buf, mask = run_gemm_ex(A, B, dtype, -1.5, 0.75, c_code, old,
                                           variant=mg.MFMA16, config=c, ta=ta, tb=tb,
                                           ldc=N + 3, c_off=1)
                check_ex(C, A, B, dtype, -1.5, 0.75, c_code, old, ref=ref)
                assert padding_untouched(buf, mask)


def test_packed_integer_inputs_exact():
    M, N, K = 150, 90, 1000
    for dtype in ("f16", "bf16"):
        A, B = inputs.pair(M, N, K, dtype, "int", seed=12)
        ref = oracle_ref(A, B, dtype)
        for ta, tb in LAYOUTS:
            for c in PACKED:
                say(f"packed int {_name(ta, tb)} {dtype} cfg={c}")
                C, _, _ = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None, variant=mg.MFMA16,
                                      config=c, ta=ta, tb=tb, lda=(M if ta else K) + 1)
                check_ex(C, A, B, dtype, 1.0, 0.0, 0, None, ref=ref, exact=True)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_auto_selects_packing_where_needed(ta, tb):
    """K = 1000 (not a multiple of 64) and an odd leading dimension: with a
    workspace lent the selection takes a packed configuration, without one the
    register-staged kernel, and both results match."""
    M, N, K = 600, 520, 1000
    lda, ldb = (M if ta else K), (K if tb else N) + 1
    st, text = mg.migemm_describe_ex(-1, -1, int(ta), int(tb), M, N, K, 1, None, lda, None, ldb,
                                     0, N, 1 << 30)
    assert st == mg.OK and mg._parse_description(text)["config"] in PACKED
    st, text = mg.migemm_describe_ex(-1, -1, int(ta), int(tb), M, N, K, 1, None, lda, None, ldb,
                                     0, N, 0)
    assert st == mg.OK and mg._parse_description(text)["config"] not in PACKED
    A, B = inputs.pair(M, N, K, "f16", "normal", seed=44 + ta + 2 * tb)
    ref = oracle_ref(A, B, "f16")
    for ws in ("auto", None):
        say(f"packed auto {_name(ta, tb)} {M}x{N}x{K} workspace={ws}")
        C, _, _ = run_gemm_ex(A, B, "f16", 1.0, 0.0, 0, None, ta=ta, tb=tb, ldb=ldb, ws=ws)
        check_ex(C, A, B, "f16", 1.0, 0.0, 0, None, ref=ref)


def test_packed_two_streams_own_workspaces():
    """Calls alternating between two streams, each lent its own workspace
    (allocated on its stream), launched back to back and checked after one
    synchronisation."""
    shapes = [(64, 72, 130), (700, 300, 513), (33, 40, 9), (512, 640, 1001), (120, 8, 70),
              (900, 257, 333)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for i, (M, N, K) in enumerate(shapes):
        dtype = ("f16", "bf16")[i % 2]
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=100 + i)
        dA, _ = to_device_with_ld(A, K + 1, 1)
        dB, _ = to_device_with_ld(B, N + 1, 1)
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        runs.append((A, B, dtype, dA, dB, C, K + 1, N + 1))
    torch.cuda.synchronize()
    keep = []
    for i, (A, B, dtype, dA, dB, C, lda, ldb) in enumerate(runs):
        M, K = A.shape
        N = B.shape[1]
        s = streams[i % 2]
        cfg = PACKED[i % 2]
        st, n = mg.migemm_workspace_size(mg.MFMA16, cfg, 0, 0, M, N, K, DT_CODE[dtype],
                                         dA.data_ptr(), lda, dB.data_ptr(), ldb)
        assert st == mg.OK and n > 0
        with torch.cuda.stream(s):
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        keep.append(ws)
        say(f"packed stream {i % 2} {dtype} {M}x{N}x{K} workspace {n}")
        st = mg.migemm_gemm_ws(mg.MFMA16, cfg, 0, 0, M, N, K, DT_CODE[dtype], dA.data_ptr(),
                               lda, dB.data_ptr(), ldb, 1.0, 0.0, 0, C.data_ptr(), N,
                               ws.data_ptr(), n, s.cuda_stream)
        assert st == mg.OK
    torch.cuda.synchronize()
    for (A, B, dtype, dA, dB, C, lda, ldb) in runs:
        check_ex(C.cpu(), A, B, dtype, 1.0, 0.0, 0, None)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_packed_without_usable_workspace_runs_in_place(dtype):
    """A packed configuration lent no workspace, one byte too little, or a
    workspace off a 256-byte boundary runs in place (register-staged kernel);
    a workspace exactly as large as asked is used, and nothing past the size
    migemm_workspace_size reports is written."""
    M, N, K = 300, 264, 200
    A, B = inputs.pair(M, N, K, dtype, "normal", seed=71)
    ref = oracle_ref(A, B, dtype)
    for cfg in PACKED:
        st, need = mg.migemm_workspace_size(mg.MFMA16, cfg, 0, 0, M, N, K, DT_CODE[dtype], None,
                                            K + 1, None, N)
        assert st == mg.OK and need > 0
        for case, ws in (("none", None), ("short", need - 1), ("exact", need)):
            say(f"packed {dtype} cfg={cfg} workspace {case}")
            C, _, _ = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None, variant=mg.MFMA16, config=cfg,
                                  lda=K + 1, ws=ws)
            check_ex(C, A, B, dtype, 1.0, 0.0, 0, None, ref=ref)
        # a misaligned workspace and a guarded one, lent directly
        dA, _ = to_device_with_ld(A, K + 1, 0)
        dB, _ = to_device_with_ld(B, N, 0)
        stream = torch.cuda.current_stream().cuda_stream
        guard = 4096
        buf = torch.full((need + 256 + guard,), 0xA5, dtype=torch.uint8, device="cuda")
        for off, label in ((16, "misaligned"), (0, "aligned")):
            C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            say(f"packed {dtype} cfg={cfg} workspace {label}")
            st = mg.migemm_gemm_ws(mg.MFMA16, cfg, 0, 0, M, N, K, DT_CODE[dtype], dA.data_ptr(),
                                   K + 1, dB.data_ptr(), N, 1.0, 0.0, 0, C.data_ptr(), N,
                                   buf.data_ptr() + off, need + 256, stream)
            torch.cuda.synchronize()
            assert st == mg.OK
            check_ex(C.cpu(), A, B, dtype, 1.0, 0.0, 0, None, ref=ref)
        tail = buf[need:].cpu()
        assert bool((tail == 0xA5).all()), "workspace written past the reported size"
        assert not bool((buf[:need].cpu() == 0xA5).all()), "aligned workspace not used"


def test_packed_last_row_band_split():
    """With the 128x128 tile, a last band of tile rows that would start a second
    round of workgroups (17 x 16 tiles for 2050 x 2047) runs as a launch of its
    own on the 64x64 tile, after the whole 128-row bands.  Cases: both operands
    packed (ragged K, odd ldb); both read in place (aligned, K a multiple of 64),
    also with A given transposed (the tail starts at a column of A); the general
    output step into 16-bit C with a padded ldc (the tail starts at a row of C);
    and the same split on the direct path (configuration 7 called on aligned
    operands)."""
    dtype = "f16"
    # (M, N, K, ta, tb, C dtype code, ldc padding, configuration): 12 packs or
    # reads in place, then runs 7; 7 on aligned operands is the direct path
    cases = [(2050, 2047, 200, False, False, 0, 0, 12),
             (2050, 2048, 256, False, False, 0, 0, 12),
             (2056, 2048, 128, True, False, 0, 0, 12),
             (2050, 2047, 136, False, True, 2, 3, 12),
             (2050, 2048, 256, False, False, 0, 0, 7),
             (2056, 2048, 192, True, False, 1, 8, 7)]
    for (M, N, K, ta, tb, c_code, pad, cfg) in cases:
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=M + N + K)
        ref = oracle_ref(A, B, dtype)
        alpha, beta = (1.0, 0.0) if c_code == 0 else (0.5, -1.0)
        old = None
        if c_code:
            old = (torch.rand((M, N), generator=torch.Generator().manual_seed(K)) - 0.5).to(
                {1: torch.float16, 2: torch.bfloat16}[c_code])
        say(f"last-band split cfg={cfg} {_name(ta, tb)} {M}x{N}x{K} c_dtype={c_code} ldc=N+{pad}")
        C, buf, mask = run_gemm_ex(A, B, dtype, alpha, beta, c_code, old, variant=mg.MFMA16,
                                   config=cfg, ta=ta, tb=tb, ldc=N + pad)
        check_ex(C, A, B, dtype, alpha, beta, c_code, old, ref=ref)
        assert padding_untouched(buf, mask)


def test_split_tail_on_the_skinny_kernel():
    """The rows past the last whole 128-row band, when they would start a second
    round of workgroups: 1 to 16 rows go to the skinny kernel (K split over the
    waves of each workgroup), more to the 64x64 tile.  Cases: 1, 4, 16 and 17 tail
    rows on the direct path; B given transposed (k-contiguous skinny loads); A
    given transposed and row-major B (k-row chunks staged through LDS); the
    general output step into FP32, FP16 and BF16 C; the packed path (ragged K);
    and a row-major B the skinny kernel cannot read in 16-byte chunks."""
    dtype = "bf16"
    # (M, N, K, ta, tb, C dtype code, configuration)
    cases = [(2049, 2048, 128, False, False, 0, 7),
             (2052, 2000, 192, False, False, 0, 7),
             (2064, 2048, 64, False, True, 0, 7),
             (2065, 2048, 128, False, False, 0, 7),
             (2056, 2040, 128, True, False, 0, 7),
             (2049, 2048, 128, False, False, 2, 7),
             (2051, 2047, 100, False, False, 0, 12),
             (2053, 2048, 96, True, True, 1, 12),
             # K a multiple of 8 but not of 32: partial last k-tile (direct) and
             # partial last k-step (skinny); sixteen-wave skinny (B given transposed)
             (2050, 2048, 136, False, False, 0, 7),
             (2050, 2048, 2056, False, True, 0, 7),
             (2050, 2047, 2056, False, False, 0, 12),
             # row-major B and A given transposed staged through LDS (16-byte
             # k-row chunks, transposing reads): sixteen tail rows of A^T, eight
             # with B k-contiguous, a single 8-deep k-step, a 16-bit C
             (2064, 2048, 2056, True, False, 0, 7),
             (2056, 2040, 128, True, True, 0, 7),
             (2049, 2048, 8, False, False, 0, 7),
             (2052, 2000, 192, False, False, 1, 7),
             # odd N, row-major B off its 16-byte boundary: the tail runs on the
             # 64x64 configuration instead
             (2050, 2047, 64, False, False, 0, 7)]
    for (M, N, K, ta, tb, c_code, cfg) in cases:
        A, B = inputs.pair(M, N, K, dtype, "normal", seed=M + 3 * N + K + ta + 2 * tb)
        ref = oracle_ref(A, B, dtype)
        alpha, beta = (1.0, 0.0) if c_code == 0 else (-0.5, 1.5)
        old = None
        if c_code:
            old = (torch.rand((M, N), generator=torch.Generator().manual_seed(K)) - 0.5).to(
                {1: torch.float16, 2: torch.bfloat16}[c_code])
        say(f"split tail cfg={cfg} {_name(ta, tb)} {M}x{N}x{K} c_dtype={c_code}")
        C, buf, mask = run_gemm_ex(A, B, dtype, alpha, beta, c_code, old, variant=mg.MFMA16,
                                   config=cfg, ta=ta, tb=tb)
        check_ex(C, A, B, dtype, alpha, beta, c_code, old, ref=ref)
        assert padding_untouched(buf, mask)
    # what runs: the main launch, then the tail on 16-column workgroups (or 64x64 tiles)
    for (M, tail_grid) in [(2049, 128), (2064, 128), (2065, 32)]:
        st, text = mg.migemm_describe_ex(mg.MFMA16, 7, 0, 0, M, 2048, 128, 2, None, 128, None,
                                         2048, 0, 2048, 0)
        d = mg._parse_description(text)
        assert st == mg.OK and d["launches"] == 2 and d["grid1"] == tail_grid, text
    # sixteen waves unless A is given transposed (eight)
    for (ta, block) in [(0, 1024), (1, 512)]:
        st, text = mg.migemm_describe_ex(mg.MFMA16, 7, ta, 0, 2056, 2048, 128, 2, None,
                                         2056 if ta else 128, None, 2048, 0, 2048, 0)
        d = mg._parse_description(text)
        assert st == mg.OK and d["launches"] == 2 and d["block1"] == block, text


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_packed_fp32_every_layout(ta, tb):
    """FP32 configuration 13: operands the direct FP32 kernel cannot read (odd
    leading dimensions, element offsets of 1 and 3, K not a multiple of 4) are
    copied into aligned images with K zero-filled to a multiple of 32, then the
    direct FP32 kernel runs on the copies; from K = 1 to past several k-tiles,
    ragged M and N, the general output step into BF16 C."""
    v = mg.REGTILE_MFMA
    for (M, N, K, pad, off) in [(1, 1, 1, 0, 0), (7, 9, 5, 0, 0), (203, 170, 301, 3, 1),
                                (300, 264, 200, 5, 3), (257, 513, 130, 0, 0)]:
        A, B = inputs.pair(M, N, K, "f32", "uniform", seed=M + 2 * N + 3 * K + 5 * ta + 7 * tb)
        ref = oracle_ref(A, B, "f32")
        lda = (M if ta else K) + pad
        ldb = (K if tb else N) + pad
        say(f"packed fp32 {_name(ta, tb)} {M}x{N}x{K} lda={lda} ldb={ldb} off={off}")
        C, buf, mask = run_gemm_ex(A, B, "f32", 1.0, 0.0, 0, None, variant=v, config=13, ta=ta,
                                   tb=tb, lda=lda, ldb=ldb, a_off=off, b_off=off)
        check_ex(C, A, B, "f32", 1.0, 0.0, 0, None, ref=ref)
        assert padding_untouched(buf, mask)
    A, B = inputs.pair(300, 264, 203, "f32", "uniform", seed=17 + ta)
    old = (torch.rand((300, 264), generator=torch.Generator().manual_seed(3)) - 0.5).to(
        torch.bfloat16)
    say(f"packed fp32 {_name(ta, tb)} general output")
    C, buf, mask = run_gemm_ex(A, B, "f32", 0.5, -1.0, 2, old, variant=v, config=13, ta=ta, tb=tb,
                               lda=(300 if ta else 203) + 1, ldb=(203 if tb else 264) + 1,
                               ldc=264 + 3)
    check_ex(C, A, B, "f32", 0.5, -1.0, 2, old)
    assert padding_untouched(buf, mask)


def test_packed_fp32_selected():
    """The selection copies FP32 operands the direct kernel cannot read once the
    product is large enough and a workspace is lent: 2049^3 (then the 128x128
    tile on the whole tiles and the skinny kernel on the last row and column)
    and 1023^3 (then the 64x64 tile)."""
    for (M, N, K) in [(2049, 2049, 2049), (1023, 1023, 1023)]:
        st, text = mg.migemm_describe_ex(-1, -1, 0, 0, M, N, K, mg.F32, None, K, None, N, 0, N,
                                         1 << 40)
        assert st == mg.OK and mg._parse_description(text)["config"] == 13, text
        A, B = inputs.pair(M, N, K, "f32", "uniform", seed=M)
        say(f"packed fp32 {M}x{N}x{K} through the selection")
        C, buf, mask = run_gemm_ex(A, B, "f32", 1.0, 0.0, 0, None)
        check_ex(C, A, B, "f32", 1.0, 0.0, 0, None)
        assert padding_untouched(buf, mask)
