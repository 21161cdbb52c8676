"""Products whose last band of tile rows or columns would start a second round of
workgroups: the whole tiles run on the requested tile shape (on the ping-pong
kernel when they are whole 256x256 or 128x256 tiles and whole k-tiles), the rows
past them on the skinny kernel (up to 16) or the 64x64 tile, and the columns past
them on the skinny kernel as the transposed product C^T = B^T A^T (up to 16,
written transposed into C) or the 64x64 tile.  Every element is compared with
the oracle, and the NaN padding around C must stay untouched.

K is kept small (64 to 136) so that the oracle finishes quickly; the split
depends only on M, N and the tile shape.  Leading dimensions are rounded up to a
multiple of 8 so that the direct kernels and the skinny kernel's 16-byte reads
apply in every layout.
"""
import pytest
import torch

import dense_gemm_16_amd as mg
from dense_gemm_16_amd import inputs
from gpu_helpers import check_ex, oracle_ref, padding_untouched, run_gemm_ex, say

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _name(ta, tb):
    return ("T" if ta else "N") + ("T" if tb else "N")


def _r8(x):
    return (x + 7) // 8 * 8


def _run(M, N, K, ta, tb, config, c_code=0, dtype="bf16", pad_c=0, seed=0, variant=mg.MFMA16,
         dist="normal", exact=False):
    A, B = inputs.pair(M, N, K, dtype, dist, seed=seed + M + 3 * N + 7 * K + ta + 2 * tb)
    ref = oracle_ref(A, B, dtype)
    alpha, beta = (1.0, 0.0) if c_code == 0 else (0.75, -1.25)
    old = None
    if c_code:
        old = (torch.rand((M, N), generator=torch.Generator().manual_seed(K)) - 0.5).to(
            {1: torch.float16, 2: torch.bfloat16}[c_code])
    lda = _r8(M if ta else K)
    ldb = _r8(K if tb else N)
    say(f"split variant={variant} cfg={config} {_name(ta, tb)} {M}x{N}x{K} {dtype} {dist} "
        f"c_dtype={c_code} lda={lda} ldb={ldb} ldc=N+{pad_c}")
    C, buf, mask = run_gemm_ex(A, B, dtype, alpha, beta, c_code, old, variant=variant,
                               config=config, ta=ta, tb=tb, lda=lda, ldb=ldb, ldc=N + pad_c)
    check_ex(C, A, B, dtype, alpha, beta, c_code, old, ref=ref, exact=exact)
    assert padding_untouched(buf, mask)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_split_rows_and_columns_every_layout(ta, tb):
    """256x256 tiles: four rows past 16 whole tile rows (the skinny kernel), eight
    columns past 16 whole tile columns (the skinny kernel on the transposed
    product, whose operand forms follow the layout: B's column slab k-contiguous
    when B is given transposed, k-rows otherwise; A likewise), and both at once;
    the whole tiles run on the ping-pong kernel."""
    _run(4100, 4096, 64, ta, tb, 10)
    _run(4096, 4104, 64, ta, tb, 10)
    _run(4100, 4104, 128, ta, tb, 10)


def test_split_wider_tails_on_the_64x64_tile():
    """Tails of more than 16 rows or columns run on the 64x64 tile."""
    _run(4160, 4096, 64, False, False, 10)
    _run(4096, 4160, 64, False, True, 10)
    _run(4120, 4136, 64, True, False, 10)


def test_split_other_tile_shapes_and_ragged_k():
    """128x128 tiles (configuration 7) with eight tail columns and a K that ends
    inside a k-tile; 128x256 tiles (configuration 13) with eight tail rows (whole
    tiles then run on its ping-pong kernel, 15) or eight tail columns and a ragged
    K (they stay on 13); the ping-pong configuration asked for on a ragged shape;
    FP16 inputs."""
    _run(2048, 2056, 136, False, False, 7)
    _run(2048, 2056, 136, True, True, 7, dtype="f16")
    _run(2056, 4096, 128, False, False, 13)
    _run(2048, 4104, 72, True, False, 13)
    _run(4100, 4096, 64, False, True, 14, dtype="f16")


def test_split_general_output():
    """alpha * A x B + beta * C into 16-bit C with a padded leading dimension: the
    transposed tail writes C element by element in its own rows and columns."""
    _run(4096, 4104, 64, False, False, 10, c_code=1, pad_c=3)
    _run(4100, 4104, 64, True, False, 10, c_code=2, pad_c=8)
    _run(2048, 2056, 64, False, True, 7, c_code=0, pad_c=5)


def test_split_after_packing():
    """Operands the direct kernel cannot read in place are copied first; the split
    then runs on the copies (B' = B^T, k-contiguous), including a column tail."""
    for (M, N, K, ta, tb, cfg) in [(2050, 2050, 100, False, False, 12),
                                   (4100, 4099, 64, False, False, 11)]:
        A, B = inputs.pair(M, N, K, "f16", "normal", seed=M + N + K)
        ref = oracle_ref(A, B, "f16")
        say(f"split after packing cfg={cfg} {M}x{N}x{K}")
        C, buf, mask = run_gemm_ex(A, B, "f16", 1.0, 0.0, 0, None, variant=mg.MFMA16,
                                   config=cfg, ta=ta, tb=tb)
        check_ex(C, A, B, "f16", 1.0, 0.0, 0, None, ref=ref)
        assert padding_untouched(buf, mask)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_split_fp32_every_layout(ta, tb):
    """FP32 on the FP32 matrix-core kernels: the 128x128 tile (configuration 10)
    with eight tail rows, eight tail columns and both, on the FP32 skinny kernel
    (16-deep k-steps of four 16x16x4 instructions; k-row operands staged through
    LDS and read back four k-rows at a time); K a multiple of 4 but not of the
    16-deep step."""
    _run(2056, 2048, 68, ta, tb, 10, dtype="f32", variant=mg.REGTILE_MFMA)
    _run(2048, 2056, 68, ta, tb, 10, dtype="f32", variant=mg.REGTILE_MFMA)
    _run(2056, 2056, 96, ta, tb, 10, dtype="f32", variant=mg.REGTILE_MFMA)


def test_split_fp32_other_cases():
    """FP32: the 64x64 tile (configuration 8) with tails of 8 rows or columns; a
    52-row tail of the 128x128 tile on the 64x64 one; the general output step into
    BF16 C; small-integer inputs, which must come out exact."""
    v = mg.REGTILE_MFMA
    _run(1032, 1024, 64, False, False, 8, dtype="f32", variant=v)
    _run(1024, 1032, 64, True, True, 8, dtype="f32", variant=v)
    _run(2100, 2048, 64, False, True, 10, dtype="f32", variant=v)
    _run(2048, 2056, 64, False, False, 10, dtype="f32", variant=v, c_code=2, pad_c=3)
    _run(2056, 2056, 64, True, False, 10, dtype="f32", variant=v, dist="int", exact=True)


def test_split_tails_ending_inside_a_chunk():
    """Tails whose k-row side ends inside a 16-byte chunk: the skinny kernel reads
    that last chunk element by element.  Three columns past the whole tiles with
    row-major B (the transposed product's left operand), four rows past them with
    A given transposed, in FP16, BF16 and FP32 (configurations asked for on
    operands with aligned, padded leading dimensions)."""
    _run(4096, 4099, 64, False, False, 10, dtype="f16")
    _run(4100, 4096, 64, True, True, 10)
    _run(4100, 4099, 64, True, False, 10)
    _run(2048, 2051, 64, False, False, 10, dtype="f32", variant=mg.REGTILE_MFMA)
    _run(2054, 2048, 64, True, True, 10, dtype="f32", variant=mg.REGTILE_MFMA)
