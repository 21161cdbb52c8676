"""Split-K (FP16/BF16 configuration 17): products whose M x N is a few 128x128
tiles and whose K is long are summed as slices of K, on the 128x128 tile or,
with 16 or more 256x256 tiles, the 256x256 one, each slice's workgroups
writing FP32 sums into the lent workspace, then a second kernel adds the
slices in order and applies the output step.  Compared element by element with
the oracle: every layout, a K that ends inside a k-tile (only the last slice is
partial), fewer slices than asked for where K runs out of whole k-tiles, the
general output step into 16-bit C with a padded leading dimension, and the long
products the selection sends here.  The result must not
depend on timing: two calls give the same bits.  Without a workspace the
configuration runs the ordinary 128x128 launch.
"""
import pytest
import torch

import dense_gemm_16_amd as mg
from dense_gemm_16_amd import inputs
from gpu_helpers import (DT_CODE, check_ex, oracle_ref, padding_untouched, run_gemm_ex, say,
                         to_device_with_ld)

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _describe(M, N, K, dtype, ta, tb, lda, ldb, ws_bytes, variant=-1, config=-1):
    st, text = mg.migemm_describe_ex(variant, config, int(ta), int(tb), M, N, K, DT_CODE[dtype],
                                     None, lda, None, ldb, 0, N, ws_bytes)
    assert st == mg.OK, text
    return mg._parse_description(text)


def _run(M, N, K, ta, tb, dtype="bf16", c_code=0, pad_c=0, config=17, seed=0, variant=mg.MFMA16):
    A, B = inputs.pair(M, N, K, dtype, "normal", seed=seed + M + 3 * N + 5 * K + ta + 2 * tb)
    ref = oracle_ref(A, B, dtype)
    alpha, beta = (1.0, 0.0) if c_code == 0 else (-0.5, 1.25)
    old = None
    if c_code:
        old = (torch.rand((M, N), generator=torch.Generator().manual_seed(K)) - 0.5).to(
            {1: torch.float16, 2: torch.bfloat16}[c_code])
    lda = M if ta else K
    ldb = K if tb else N
    say(f"splitk cfg={config} {'T' if ta else 'N'}{'T' if tb else 'N'} {M}x{N}x{K} {dtype} "
        f"c_dtype={c_code} ldc=N+{pad_c}")
    C, buf, mask = run_gemm_ex(A, B, dtype, alpha, beta, c_code, old, variant=variant,
                               config=config, ta=ta, tb=tb, lda=lda, ldb=ldb, ldc=N + pad_c)
    check_ex(C, A, B, dtype, alpha, beta, c_code, old, ref=ref)
    assert padding_untouched(buf, mask)
    return C


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_splitk_every_layout(ta, tb):
    """256 x 256 x 16384: four tiles, 16 slices of 1024."""
    d = _describe(256, 256, 16384, "bf16", ta, tb, 256 if ta else 16384, 16384 if tb else 256,
                  1 << 30)
    assert d["config"] == 17 and d["launches"] == 2 and d["grid0"] == 4 * 16
    _run(256, 256, 16384, ta, tb)


def test_splitk_ragged_k_and_fewer_slices():
    """K = 8200 over 6 tiles: slices of 576, 15 of them, the last 136 deep (a
    partial k-tile); K = 4160 on one tile: slices of 320, 13 of them; FP16 and
    BF16, row and column counts that are not whole tiles, and an M x N that is
    not a multiple of 4 (the sum kernel then adds element by element)."""
    _run(264, 200, 8200, False, False)
    _run(264, 200, 8200, True, True, dtype="f16")
    _run(128, 128, 4160, False, True, dtype="f16")
    _run(72, 40, 4104, True, False)
    # M x N not a multiple of 4: the sum kernel's element-wise path
    _run(263, 199, 8200, False, True)


def test_splitk_256x256_tile():
    """The slices on the 256x256 tile (configuration 10): 16 tiles in 16 slices of
    4096; 42 tiles (the 128x128 tile's 156 would overshoot a round in two
    slices) in 6 slices of 1408 whose last is 1160 deep (a partial first k-tile
    in that slice only); a ragged N with B given transposed; the general output
    step into BF16 C."""
    for (M, N, K, ta, tb, grid) in [(1024, 1024, 65536, False, False, 16 * 16),
                                    (1544, 1536, 8200, True, False, 42 * 6),
                                    (1536, 1543, 8192, False, True, 42 * 6)]:
        d = _describe(M, N, K, "bf16", ta, tb, M if ta else K, K if tb else N, 1 << 40,
                      mg.MFMA16, 17)
        assert d["launches"] == 2 and d["grid0"] == grid, d
        _run(M, N, K, ta, tb)
    _run(1536, 1536, 8192, True, True, dtype="f16", c_code=2, pad_c=8)


def test_splitk_general_output():
    """alpha * A x B + beta * C into FP16 and BF16 C with padded rows: the sum
    kernel applies the output step to the total of the slices."""
    _run(512, 384, 4096, False, False, c_code=1, pad_c=5)
    _run(200, 328, 8192, True, False, dtype="f16", c_code=2, pad_c=8)
    _run(384, 256, 4096, False, True, c_code=0, pad_c=3)


def test_splitk_without_workspace_runs_the_128x128_launch():
    A, B = inputs.pair(256, 256, 8192, "bf16", "normal", seed=11)
    say("splitk cfg=17 without a workspace")
    C, buf, mask = run_gemm_ex(A, B, "bf16", 1.0, 0.0, 0, None, variant=mg.MFMA16, config=17,
                               ws=None)
    check_ex(C, A, B, "bf16", 1.0, 0.0, 0, None)
    assert padding_untouched(buf, mask)


def test_splitk_same_bits_twice():
    """The slices are added in a fixed order: two calls, the workspace poisoned in
    between, give identical bits."""
    M, N, K = 384, 256, 16384
    A, B = inputs.pair(M, N, K, "f16", "normal", seed=12)
    dA, _ = to_device_with_ld(A, K, 0)
    dB, _ = to_device_with_ld(B, N, 0)
    st, need = mg.migemm_workspace_size(-1, -1, 0, 0, M, N, K, 1, dA.data_ptr(), K,
                                        dB.data_ptr(), N)
    assert st == mg.OK and need == 16 * M * N * 4
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    for r in range(2):
        ws.fill_(0xFF)  # NaN in every FP32 slot
        C = torch.full((M, N), float("nan"), device="cuda")
        say(f"splitk same bits: call {r}")
        st = mg.migemm_gemm_ws(-1, -1, 0, 0, M, N, K, 1, dA.data_ptr(), K, dB.data_ptr(), N,
                               1.0, 0.0, 0, C.data_ptr(), N, ws.data_ptr(), need, stream)
        assert st == mg.OK
        torch.cuda.synchronize()
        out.append(C.cpu())
    assert torch.equal(out[0].view(torch.int32), out[1].view(torch.int32))
    check_ex(out[0], A, B, "f16", 1.0, 0.0, 0, None)


@pytest.mark.parametrize("M,N,K,dtype", [(512, 512, 65536, "bf16"), (1024, 1024, 65536, "f16"),
                                         (64, 64, 65536, "bf16"), (1000, 1016, 8200, "bf16")])
def test_splitk_long_products(M, N, K, dtype):
    """The long products the selection sends to split-K (16 slices of 4096; 4 of
    16384; one tile in 16 slices; 64 tiles with a partial last k-tile), through
    the automatic selection with the workspace it asks for; every element."""
    d = _describe(M, N, K, dtype, False, False, K, N, 1 << 40)
    assert d["config"] == 17, d
    A, B = inputs.pair(M, N, K, dtype, "normal", seed=M + N + K)
    say(f"splitk {M}x{N}x{K} {dtype} through the selection")
    C, buf, mask = run_gemm_ex(A, B, dtype, 1.0, 0.0, 0, None)
    check_ex(C, A, B, dtype, 1.0, 0.0, 0, None)
    assert padding_untouched(buf, mask)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_splitk_fp32_every_layout(ta, tb):
    """FP32 split-K (configuration 12 of the FP32 matrix-core variant): slices on
    the direct 64x64 FP32 tile; 256 x 256 x 16384 is 16 tiles in 16 slices of
    1024."""
    v = mg.REGTILE_MFMA
    d = _describe(256, 256, 16384, "f32", ta, tb, 256 if ta else 16384, 16384 if tb else 256,
                  1 << 30, v, 12)
    assert d["launches"] == 2 and d["grid0"] == 16 * 16, d
    _run(256, 256, 16384, ta, tb, dtype="f32", config=12, variant=v)


def test_splitk_fp32_ragged_and_general():
    """FP32: K a multiple of 4 but not of the 32-deep k-tile (only the last slice
    ends inside one), ragged M and N, the general output step into BF16 C with a
    padded leading dimension, and the selection's own choice on a long product."""
    v = mg.REGTILE_MFMA
    _run(264, 200, 8196, False, False, dtype="f32", config=12, variant=v)
    _run(200, 264, 8196, True, True, dtype="f32", config=12, variant=v)
    _run(256, 192, 8192, False, True, dtype="f32", c_code=2, pad_c=8, config=12, variant=v)
    d = _describe(512, 512, 65536, "f32", False, False, 65536, 512, 1 << 40)
    assert d["variant"] == "regtile_mfma" and d["config"] == 12, d
    A, B = inputs.pair(512, 512, 65536, "f32", "uniform", seed=13)
    say("splitk fp32 512x512x65536 through the selection")
    C, buf, mask = run_gemm_ex(A, B, "f32", 1.0, 0.0, 0, None)
    check_ex(C, A, B, "f32", 1.0, 0.0, 0, None)
    assert padding_untouched(buf, mask)
