"""Device-side element-type conversion (migemm_convert) against the oracle's
decoders and round-to-nearest-even encoders (both pinned in test_oracle.py).

Bit-exact: every 16-bit source pattern into every target, random and special
FP32 patterns (subnormals, infinities, NaN, ties, overflow thresholds), padded
and misaligned rows (padding untouched), a full 8192 x 8192 FP32 -> BF16 matrix
on sampled rows, and the conversion feeding the 16-bit product.
"""
import numpy as np
import pytest
import torch

import dense_gemm_16_amd as mg
import oracle
from dense_gemm_16_amd import inputs
from gpu_helpers import check, run_gemm, say

pytestmark = pytest.mark.gpu

TORCH_OF = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}
NAMES = {0: "f32", 1: "f16", 2: "bf16"}


def _bits(t):
    """Stored bits of a CPU tensor as a numpy array (uint32 for FP32, uint16 else)."""
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def _from_bits(b, code):
    b = np.ascontiguousarray(b)
    if code == 0:
        return torch.from_numpy(b.view(np.int32).copy()).view(torch.float32)
    return torch.from_numpy(b.view(np.int16).copy()).view(TORCH_OF[code])


def _convert(src_cpu, dst_code, lds=None, ldd=None, s_off=0, d_off=0):
    """Run migemm_convert on a copy of src inside NaN-padded buffers; returns
    (dst window on the CPU, dst buffer on the CPU, window mask)."""
    rows, cols = src_cpu.shape
    lds = lds or max(cols, 1)
    ldd = ldd or max(cols, 1)
    sbuf = torch.full((s_off + max(rows, 1) * lds + 16,), float("nan"), dtype=src_cpu.dtype,
                      device="cuda")
    sv = sbuf[s_off:s_off + rows * lds].view(rows, lds)[:, :cols]
    sv.copy_(src_cpu.to("cuda"))
    dbuf = torch.full((d_off + max(rows, 1) * ldd + 16,), float("nan"), dtype=TORCH_OF[dst_code],
                      device="cuda")
    dv = dbuf[d_off:d_off + rows * ldd].view(rows, ldd)[:, :cols]
    src_code = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[src_cpu.dtype]
    st = mg.migemm_convert(src_code, dst_code, rows, cols, sv.data_ptr(), lds, dv.data_ptr(), ldd,
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mg.OK, mg.migemm_status_string(st)
    mask = torch.zeros(dbuf.shape, dtype=torch.bool)
    mask[d_off:d_off + rows * ldd].view(rows, ldd)[:, :cols] = True
    return dv.cpu(), dbuf.cpu(), mask


def _want(src_bits, src_code, dst_code):
    return oracle.encode(oracle.decode(src_bits, src_code), dst_code)


def _assert_bits_equal(got_t, want, src_vals):
    got = _bits(got_t).reshape(-1)
    want = np.asarray(want).reshape(-1)
    if want.dtype == np.float32:
        want = want.view(np.uint32)
    nan = np.isnan(src_vals.reshape(-1))
    got_nan = np.isnan(got_t.reshape(-1).float().numpy())
    assert np.array_equal(got_nan, nan), "NaN must map to NaN and nothing else"
    bad = np.flatnonzero((got != want) & ~nan)
    assert bad.size == 0, (f"{bad.size} differ; first index {bad[0]}: source {src_vals.reshape(-1)[bad[0]]!r} "
                           f"got {got[bad[0]]:#x} want {want[bad[0]]:#x}")


@pytest.mark.parametrize("src_code", [1, 2])
@pytest.mark.parametrize("dst_code", [0, 1, 2])
def test_every_16bit_pattern(src_code, dst_code):
    pats = np.arange(65536, dtype=np.uint16).reshape(256, 256)
    src = _from_bits(pats, src_code)
    say(f"convert all patterns {NAMES[src_code]} -> {NAMES[dst_code]}")
    got, _, _ = _convert(src, dst_code)
    _assert_bits_equal(got, _want(pats, src_code, dst_code), oracle.decode(pats, src_code))


def _f32_patterns():
    g = np.random.default_rng(21)
    w = g.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    special = []
    # FP16 and BF16 midpoints (ties) and their neighbours, overflow thresholds
    for code in (1, 2):
        lo = np.arange(0, 0x7BFF if code == 1 else 0x7F7F, 37, dtype=np.uint16)
        mid = (oracle.decode(lo, code) + oracle.decode(lo + 1, code)) / 2
        special.append(mid.astype(np.float32).view(np.uint32))
    special.append(np.array([65504, 65519, 65520, 65536, 3.3895314e38, 3.3961776e38],
                            dtype=np.float32).view(np.uint32))
    special.append(np.array([0, 0x80000000, 1, 0x807FFFFF, 0x00800000, 0x7F800000, 0xFF800000,
                             0x7FC00000, 0x33000000, 0x33000001, 0x387FC000], dtype=np.uint32))
    w = np.concatenate([w] + special)
    return np.concatenate([w, np.zeros((-w.size) % 1024, dtype=np.uint32)]).reshape(-1, 1024)


@pytest.mark.parametrize("dst_code", [0, 1, 2])
def test_fp32_patterns(dst_code):
    pats = _f32_patterns()
    src = _from_bits(pats, 0)
    say(f"convert f32 patterns -> {NAMES[dst_code]}")
    got, _, _ = _convert(src, dst_code)
    _assert_bits_equal(got, _want(pats, 0, dst_code), src.numpy())


@pytest.mark.parametrize("src_code,dst_code", [(0, 2), (0, 1), (2, 0), (1, 2)])
def test_padded_and_misaligned_rows(src_code, dst_code):
    rows, cols = 37, 203
    g = torch.Generator().manual_seed(src_code * 3 + dst_code)
    src = (torch.randn(rows, cols, generator=g) * 100).to(TORCH_OF[src_code])
    for lds, ldd, s_off, d_off in [(cols, cols, 0, 0), (cols + 13, cols + 5, 0, 0),
                                   (208, 216, 0, 0), (208, 216, 1, 3)]:
        say(f"convert padded {NAMES[src_code]} -> {NAMES[dst_code]} lds={lds} ldd={ldd} off={s_off},{d_off}")
        got, dbuf, mask = _convert(src, dst_code, lds, ldd, s_off, d_off)
        _assert_bits_equal(got, _want(_bits(src), src_code, dst_code), src.float().numpy())
        assert torch.isnan(dbuf[~mask].float()).all(), "padding written"


def test_large_fp32_to_bf16_sampled_rows():
    n = 8192
    g = torch.Generator().manual_seed(4)
    src = torch.randn(n, n, generator=g)
    say("convert 8192x8192 f32 -> bf16")
    got, _, _ = _convert(src, 2)
    rows = np.random.default_rng(1).integers(0, n, 64)
    for r in list(rows) + [0, n - 1]:
        _assert_bits_equal(got[r:r + 1], _want(_bits(src[r:r + 1]), 0, 2), src[r:r + 1].numpy())


@pytest.mark.parametrize("dst", ["f16", "bf16"])
def test_conversion_feeds_the_16bit_product(dst):
    """FP32 data converted on the device, then the 16-bit product: equal to the
    oracle's product of the host-rounded operands (the conversion is exact to the
    oracle's encoder, so the parity bar is the product's own)."""
    M, N, K = 300, 264, 256
    code = {"f16": 1, "bf16": 2}[dst]
    g = torch.Generator().manual_seed(9)
    A32, B32 = torch.randn(M, K, generator=g), torch.randn(K, N, generator=g)
    say(f"convert then product {dst}")
    a = mg.convert(A32.cuda(), TORCH_OF[code])
    b = mg.convert(B32.cuda(), TORCH_OF[code])
    torch.cuda.synchronize()
    A16 = _from_bits(_want(_bits(A32), 0, code), code)
    B16 = _from_bits(_want(_bits(B32), 0, code), code)
    assert torch.equal(a.cpu().view(torch.int16), A16.view(torch.int16))
    C, _ = run_gemm(A16, B16, dst)
    check(C, A16, B16, dst)
