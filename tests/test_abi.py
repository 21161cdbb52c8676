"""The C-ABI library loads, exports what include/migemm.h declares, and checks its
arguments before touching the GPU (CPU only: no call here launches a kernel)."""
import ctypes
import os
import re

import pytest

import dense_gemm_16_amd as mg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "migemm.h")

# Device pointers are never dereferenced on these paths; any non-null value will do.
P = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(migemm_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 11
    lib = mg.lib()
    for n in names:
        assert hasattr(lib, n), f"libmigemm.so does not export {n}"
    assert sorted(mg.EXPORTS) == names


def test_exports_are_c_symbols():
    # extern "C": the dynamic symbol table holds the plain names
    cdll = ctypes.CDLL(mg.LIBRARY_PATH)
    for n in declared_functions():
        getattr(cdll, n)


def test_variant_registry():
    assert mg.migemm_variant_count() == 6
    names = [mg.migemm_variant_name(v) for v in range(6)]
    assert names == ["naive", "lds_tiled", "regtile_valu", "regtile_mfma", "mfma16", "mfma_i8"]
    assert mg.migemm_variant_name(6) is None and mg.migemm_variant_name(-1) is None
    assert all(mg.migemm_variant_supports(mg.NAIVE, d) for d in (0, 1, 2))
    assert mg.migemm_variant_supports(mg.MFMA_I8, mg.I8)
    assert not any(mg.migemm_variant_supports(mg.MFMA_I8, d) for d in (0, 1, 2))
    assert not any(mg.migemm_variant_supports(v, mg.I8) for v in range(5))
    assert not mg.migemm_variant_supports(mg.NAIVE, mg.I32)
    for v in (mg.LDS_TILED, mg.REGTILE_VALU, mg.REGTILE_MFMA):
        assert mg.migemm_variant_supports(v, 0)
        assert not mg.migemm_variant_supports(v, 1) and not mg.migemm_variant_supports(v, 2)
    assert not mg.migemm_variant_supports(mg.MFMA16, 0)
    assert mg.migemm_variant_supports(mg.MFMA16, 1) and mg.migemm_variant_supports(mg.MFMA16, 2)
    for v in range(6):
        n = mg.migemm_config_count(v)
        assert n >= 1
        assert all(mg.migemm_config_name(v, c) for c in range(n))
        assert mg.migemm_config_name(v, n) is None
    assert mg.migemm_config_count(9) == 0
    assert mg.migemm_version() >= 100


def test_status_strings():
    assert mg.migemm_status_string(mg.OK) == "ok"
    for s in (1, 2, 3, 4, 77):
        assert mg.migemm_status_string(s)
    assert "scratch" in mg.migemm_status_string(mg.ERR_WORKSPACE)


def test_extent_beyond_address_space_rejected():
    # M = 2^31 - 1 rows of FP32 with lda = 2^32 - 1 span about 2^65 bytes: counted
    # in 64 bits the extent would wrap and could pass the overlap check
    big = (1 << 31) - 1
    st = mg.migemm_gemm(big, 1, 1, 0, P, (1 << 32) - 1, 2 * P, 1, 3 * P, 1, None)
    assert st == mg.ERR_INVALID_ARG
    st = mg.migemm_gemm_ex(1, 0, 1, 1, big, 0, P, (1 << 32) - 1, 2 * P, 1, 1.0, 0.0, 0, 3 * P, 1,
                           None)
    assert st == mg.ERR_INVALID_ARG
    # an extent that fits but ends past the top of the address space
    st = mg.migemm_gemm(2, 1, 1 << 20, 0, (1 << 64) - (1 << 20), 1 << 20, 2 * P, 1, 3 * P, 1, None)
    assert st == mg.ERR_INVALID_ARG


def test_leading_dimension_limit():
    # leading dimensions must be below 2^32
    for ld in ((1 << 32), (1 << 32) + 1):
        assert mg.migemm_gemm(1, 1, 1, 0, P, ld, 2 * P, 1, 3 * P, 1, None) == mg.ERR_INVALID_ARG
        assert mg.migemm_gemm(1, 1, 1, 0, P, 1, 2 * P, ld, 3 * P, 1, None) == mg.ERR_INVALID_ARG
        assert mg.migemm_gemm(1, 1, 1, 0, P, 1, 2 * P, 1, 3 * P, ld, None) == mg.ERR_INVALID_ARG
    st, v, c = mg.migemm_select(1, 1, 1, 0, None, (1 << 32) - 1, None, 1, None, 1)
    assert st == mg.OK


@pytest.mark.parametrize("args", [
    dict(M=-1), dict(N=-1), dict(K=-1), dict(dtype=3), dict(dtype=-1),
    dict(lda=3), dict(ldb=4), dict(ldc=4), dict(M=1 << 31), dict(lda=(1 << 32) + 1),
    dict(A=None), dict(B=None), dict(C=None),
])
def test_invalid_arguments_rejected_before_any_launch(args):
    a = dict(M=8, N=5, K=4, dtype=0, A=P, lda=4, B=2 * P, ldb=5, C=3 * P, ldc=5)
    a.update(args)
    st = mg.migemm_gemm(a["M"], a["N"], a["K"], a["dtype"], a["A"], a["lda"], a["B"], a["ldb"],
                        a["C"], a["ldc"], None)
    assert st == mg.ERR_INVALID_ARG


def test_overlapping_output_rejected():
    # C's byte range overlaps A's
    st = mg.migemm_gemm(16, 16, 16, 0, P, 16, 2 * P, 16, P + 64, 16, None)
    assert st == mg.ERR_INVALID_ARG
    st = mg.migemm_gemm(16, 16, 16, 1, P, 16, 2 * P, 16, 2 * P + 100, 16, None)
    assert st == mg.ERR_INVALID_ARG


@pytest.mark.parametrize("args", [
    dict(c_dtype=3), dict(c_dtype=-1), dict(dtype=5), dict(ldc=4), dict(C=None), dict(M=-2),
    dict(op_a=2), dict(op_b=-1),
    # given transposed, A is stored K x M (lda >= M = 8) and B N x K (ldb >= K = 4)
    dict(op_a=1, lda=7), dict(op_b=1, ldb=3),
])
def test_general_form_invalid_arguments(args):
    a = dict(M=8, N=5, K=4, dtype=1, A=P, lda=4, B=2 * P, ldb=5, alpha=1.5, beta=0.5, c_dtype=2,
             C=3 * P, ldc=5)
    a.update(args)
    st = mg.migemm_gemm_ex(a.get("op_a", 0), a.get("op_b", 0), a["M"], a["N"], a["K"], a["dtype"],
                           a["A"], a["lda"], a["B"], a["ldb"], a["alpha"], a["beta"],
                           a["c_dtype"], a["C"], a["ldc"], None)
    assert st == mg.ERR_INVALID_ARG
    st = mg.migemm_gemm_ex_variant(mg.NAIVE, 0, a.get("op_a", 0), a.get("op_b", 0), a["M"],
                                   a["N"], a["K"], a["dtype"], a["A"], a["lda"], a["B"],
                                   a["ldb"], a["alpha"], a["beta"], a["c_dtype"], a["C"],
                                   a["ldc"], None)
    assert st == mg.ERR_INVALID_ARG


def test_general_form_overlap_uses_output_element_size():
    # a 16 x 16 C spans 512 bytes as BF16 and 1024 as FP32: starting 400 (BF16) or
    # 1000 (FP32) bytes before A, it reaches into A
    st = mg.migemm_gemm_ex(0, 0, 16, 16, 16, 1, P, 16, 2 * P, 16, 1.0, 0.0, 2, P - 400, 16, None)
    assert st == mg.ERR_INVALID_ARG
    st = mg.migemm_gemm_ex(0, 0, 16, 16, 16, 1, P, 16, 2 * P, 16, 1.0, 0.0, 0, P - 1000, 16, None)
    assert st == mg.ERR_INVALID_ARG


def test_transposed_operand_extent_in_overlap_check():
    # A given transposed (M = 8, K = 40, lda = 100) is stored K x M and spans
    # 39 * 100 + 8 = 3908 FP16 elements (7816 bytes); read as M x K it would span
    # only 7 * 100 + 40 = 740.  A C starting 3000 bytes after A overlaps the
    # stored extent only.
    st = mg.migemm_gemm_ex(1, 0, 8, 4, 40, 1, P, 100, 3 * P, 4, 1.0, 0.0, 0, P + 3000, 4, None)
    assert st == mg.ERR_INVALID_ARG


def test_general_form_forced_variant_checks():
    f16 = (0, 1, 64, 64, 64, 1, P, 64, 2 * P, 64, 2.0, 1.0, 1, 3 * P, 64, None)
    assert mg.migemm_gemm_ex_variant(mg.LDS_TILED, -1, *f16) == mg.ERR_UNSUPPORTED
    assert mg.migemm_gemm_ex_variant(9, -1, *f16) == mg.ERR_INVALID_ARG
    assert mg.migemm_gemm_ex_variant(mg.MFMA16, 999, *f16) == mg.ERR_INVALID_ARG


@pytest.mark.parametrize("args", [
    dict(src_dtype=3), dict(dst_dtype=-1), dict(rows=-1), dict(cols=-1), dict(lds=9),
    dict(ldd=9), dict(src=None), dict(dst=None), dict(rows=1 << 31), dict(lds=1 << 32),
    dict(ldd=1 << 32),
    dict(dst=P + 100),  # overlaps src (8 x 10 FP32 from P spans 320 bytes)
])
def test_convert_invalid_arguments(args):
    a = dict(src_dtype=0, dst_dtype=2, rows=8, cols=10, src=P, lds=10, dst=3 * P, ldd=10)
    a.update(args)
    st = mg.migemm_convert(a["src_dtype"], a["dst_dtype"], a["rows"], a["cols"], a["src"],
                           a["lds"], a["dst"], a["ldd"], None)
    assert st == mg.ERR_INVALID_ARG


def test_convert_empty_is_a_noop():
    assert mg.migemm_convert(0, 1, 0, 10, None, 10, None, 10, None) == mg.OK
    assert mg.migemm_convert(2, 0, 5, 0, None, 1, None, 1, None) == mg.OK


@pytest.mark.parametrize("args,status", [
    (dict(c_dtype=0), "invalid"),            # INT8 inputs need INT32 C
    (dict(dtype=1), "invalid"),              # INT32 C needs INT8 inputs
    (dict(K=1 << 17, lda=1 << 17), "invalid"),  # 2^17 products of 2^14 reach 2^31
    (dict(alpha=2.0), "unsupported"),        # INT32 C: plain product only
    (dict(beta=1.0), "unsupported"),
])
def test_int8_argument_rules(args, status):
    a = dict(M=8, N=16, K=64, dtype=3, A=P, lda=64, B=2 * P, ldb=16, alpha=1.0, beta=0.0,
             c_dtype=4, C=3 * P, ldc=16)
    a.update(args)
    st = mg.migemm_gemm_ex(0, 0, a["M"], a["N"], a["K"], a["dtype"], a["A"], a["lda"], a["B"],
                           a["ldb"], a["alpha"], a["beta"], a["c_dtype"], a["C"], a["ldc"], None)
    assert st == {"invalid": mg.ERR_INVALID_ARG, "unsupported": mg.ERR_UNSUPPORTED}[status]


def test_int8_selection():
    st, v, c = mg.migemm_select(8192, 8192, 8192, mg.I8, None, 8192, None, 8192, None, 8192)
    assert st == mg.OK and v == mg.MFMA_I8 and mg.migemm_config_name(v, c)
    st, v, c = mg.migemm_select(64, 64, 64, mg.I8, None, 64, None, 64, None, 64)
    assert st == mg.OK and v == mg.MFMA_I8
    # whole 256 x 256 tiles, K a multiple of 128, 16-byte rows: the direct ping-pong
    # configuration; a leading dimension of half a chunk sends it to the register-staged one
    # (without a workspace); K a multiple of 16 only: the interleaved direct kernel, which
    # takes a partial first k-tile
    assert mg.migemm_select(8192, 8192, 8192, mg.I8, None, 8192, None, 8192, None, 8192)[2] == 4
    assert mg.migemm_select(8192, 8192, 8192, mg.I8, None, 8192, None, 8200, None, 8192)[2] == 3
    assert mg.migemm_select(8192, 8192, 8000, mg.I8, None, 8000, None, 8192, None, 8192)[2] == 6
    assert mg.migemm_select(8192, 8192, 8008, mg.I8, None, 8008, None, 8192, None, 8192)[2] == 3
    # below a round of 256x256 tiles, large, last bands wider than 16: configuration 6;
    # at most 16: the split (whole tiles on the ping-pong kernel, the bands after them)
    assert mg.migemm_select(2000, 2000, 2048, mg.I8, None, 2048, None, 2000, None, 2000)[2] == 6
    assert mg.migemm_select(2056, 2048, 2048, mg.I8, None, 2048, None, 2048, None, 2048)[2] == 3
    assert mg.migemm_select(1536, 1536, 1536, mg.I8, None, 1536, None, 1536, None, 1536)[2] == 2


def test_empty_output_is_a_noop():
    # M == 0 or N == 0: OK with no HIP call (null pointers allowed where there is no data)
    assert mg.migemm_gemm(0, 5, 7, 0, None, 7, P, 5, None, 5, None) == mg.OK
    assert mg.migemm_gemm(4, 0, 7, 2, P, 7, None, 1, None, 1, None) == mg.OK


def test_forced_variant_checks():
    base = (64, 64, 64, 1, P, 64, 2 * P, 64, 3 * P, 64, None)
    assert mg.migemm_gemm_variant(mg.LDS_TILED, -1, *base) == mg.ERR_UNSUPPORTED
    assert mg.migemm_gemm_variant(mg.REGTILE_MFMA, 0, *base) == mg.ERR_UNSUPPORTED
    f32 = (64, 64, 64, 0, P, 64, 2 * P, 64, 3 * P, 64, None)
    assert mg.migemm_gemm_variant(mg.MFMA16, -1, *f32) == mg.ERR_UNSUPPORTED
    assert mg.migemm_gemm_variant(7, -1, *f32) == mg.ERR_INVALID_ARG
    assert mg.migemm_gemm_variant(mg.NAIVE, 99, *f32) == mg.ERR_INVALID_ARG
    assert mg.migemm_gemm_variant(mg.VARIANT_AUTO, 0, *f32) == mg.ERR_INVALID_ARG


def test_selection_is_deterministic_and_valid():
    for (M, N, K, dt) in [(256, 256, 256, 1), (1024, 1024, 1024, 0), (1024, 1024, 1024, 1),
                          (2048, 2048, 2048, 2), (2050, 2047, 2056, 1), (8192, 8192, 8192, 2),
                          (4096, 4096, 4096, 0), (1, 1, 1, 0), (3, 100000, 7, 2)]:
        st, v, c = mg.migemm_select(M, N, K, dt, None, max(K, 1), None, N, None, N)
        assert st == mg.OK
        assert mg.migemm_variant_supports(v, dt)
        assert 0 <= c < mg.migemm_config_count(v)
        assert mg.migemm_select(M, N, K, dt, None, max(K, 1), None, N, None, N) == (st, v, c)
    st, _, _ = mg.migemm_select(4, 4, 4, 9, None, 4, None, 4, None, 4)
    assert st == mg.ERR_INVALID_ARG


def _selected(M, N, K, dt, lda, ldb, ws_bytes, op_a=0, op_b=0):
    st, text = mg.migemm_describe_ex(-1, -1, op_a, op_b, M, N, K, dt, None, lda, None, ldb,
                                     0, N, ws_bytes)
    assert st == mg.OK, text
    d = mg._parse_description(text)
    return d["variant"], d["config"]


def test_selection_packs_unreadable_16bit_operands():
    """FP16/BF16 operands the direct kernel cannot read in place (an odd
    leading dimension, K not a multiple of 8) go to the packed configurations
    once the product is large enough and a large enough workspace is lent;
    without one, or when small, they stay on the register-staged kernel, and
    aligned ones on the direct kernel (K a multiple of 8 is enough for the
    configurations that zero-fill a partial last k-tile)."""
    sel = lambda M, N, K, dt, lda, ldb: mg.migemm_select(M, N, K, dt, None, lda, None, ldb, None, N)
    big = 1 << 40
    assert _selected(2050, 2047, 2056, 1, 2056, 2047, big) == ("mfma16", 12)
    # aligned with K = 8200: the 256x256 direct kernel reads it in place, its
    # first k-tile the partial one; with an odd ldb the copies are padded to
    # K' = 8256 for the 256x256 ping-pong kernel
    assert _selected(8192, 8192, 8200, 2, 8200, 8192, big) == ("mfma16", 10)
    assert _selected(8192, 8192, 8200, 2, 8200, 8193, big) == ("mfma16", 11)
    assert _selected(2048, 2048, 2056, 2, 2056, 2048, big) == ("mfma16", 7)
    assert _selected(4096, 4096, 4096, 2, 4096, 4097, big) == ("mfma16", 11)
    # no workspace (migemm_gemm, migemm_select) or too little: register-staged
    assert sel(2050, 2047, 2056, 1, 2056, 2047) == (mg.OK, mg.MFMA16, 2)
    assert _selected(2050, 2047, 2056, 1, 2056, 2047, 17305727) == ("mfma16", 2)
    assert _selected(2050, 2047, 2056, 1, 2056, 2047, 17305728) == ("mfma16", 12)
    assert sel(4096, 4096, 4096, 2, 4096, 4097) == (mg.OK, mg.MFMA16, 2)
    assert sel(2048, 2048, 2048, 2, 2048, 2048) == (mg.OK, mg.MFMA16, 7)
    # whole 256x256 tiles take the ping-pong configuration, other shapes with as
    # many tiles the early-load one
    assert sel(8192, 8192, 8192, 2, 8192, 8192) == (mg.OK, mg.MFMA16, 14)
    assert sel(8192, 8200, 8192, 2, 8192, 8200) == (mg.OK, mg.MFMA16, 10)
    assert sel(8000, 8192, 8192, 2, 8192, 8192) == (mg.OK, mg.MFMA16, 10)
    assert sel(1024, 8192, 8192, 2, 8192, 8192) == (mg.OK, mg.MFMA16, 15)
    assert sel(4096, 2048, 8192, 1, 8192, 2048) == (mg.OK, mg.MFMA16, 15)
    assert sel(1000, 8192, 8192, 2, 8192, 8192) == (mg.OK, mg.MFMA16, 13)
    assert sel(4096, 4096, 4096, 2, 4096, 4096) == (mg.OK, mg.MFMA16, 14)
    assert sel(100, 100, 100, 1, 100, 100) == (mg.OK, mg.MFMA16, 3)
    # at most 128 tiles of 128x128: the 64x64 direct tile; 129 to 255: one partial
    # round of the 128x128 tile (the 64x64 one would take 3 or 4 rounds)
    assert sel(1024, 1024, 1024, 1, 1024, 1024) == (mg.OK, mg.MFMA16, 16)
    assert sel(256, 256, 256, 1, 256, 256) == (mg.OK, mg.MFMA16, 16)
    assert sel(2048, 1024, 2048, 1, 2048, 1024) == (mg.OK, mg.MFMA16, 16)  # 128 tiles
    assert sel(2048, 1032, 2048, 1, 2048, 1032) == (mg.OK, mg.MFMA16, 7)   # 144 tiles
    assert sel(1536, 1536, 1536, 2, 1536, 1536) == (mg.OK, mg.MFMA16, 7)
    assert sel(1792, 1792, 4096, 2, 4096, 1792) == (mg.OK, mg.MFMA16, 7)
    assert sel(2048, 2048, 2048, 0, 2049, 2048)[1] == mg.REGTILE_MFMA
    # aligned operands need no workspace: lending one changes nothing
    assert _selected(8192, 8192, 8192, 2, 8192, 8192, big) == ("mfma16", 14)


def test_selection_split_k():
    """FP16/BF16 products of fewer than 256 tiles of 128x128 with K at least 6144
    and 4 max(M, N) run as slices of K (configuration 17) when a workspace for
    the slices' FP32 sums is lent: slices x M x N x 4 bytes, as many slices as
    fill a round of 256 workgroups (2 to 16), fewer where K runs out of whole
    64-deep k-tiles; otherwise the 64x64 tile."""
    big = 1 << 40
    sel = lambda M, N, K: mg.migemm_select(M, N, K, mg.BF16, None, K, None, N, None, N)
    assert _selected(512, 512, 65536, 2, 65536, 512, big) == ("mfma16", 17)
    assert sel(512, 512, 65536) == (mg.OK, mg.MFMA16, 16)  # no workspace
    assert _selected(512, 512, 65536, 2, 65536, 512, 16 * 512 * 512 * 4) == ("mfma16", 17)
    assert _selected(512, 512, 65536, 2, 65536, 512, 16 * 512 * 512 * 4 - 1) == ("mfma16", 16)
    assert _selected(1024, 1024, 6144, 1, 6144, 1024, big) == ("mfma16", 17)
    assert _selected(1024, 1024, 6136, 1, 6136, 1024, big) == ("mfma16", 16)  # K < 6144
    assert _selected(2048, 1024, 8184, 1, 8184, 1024, big) == ("mfma16", 16)  # K < 4 max(M, N)
    assert _selected(2048, 2048, 65536, 1, 65536, 2048, big) == ("mfma16", 7)  # 256 tiles
    assert _selected(512, 512, 65540, 1, 65540, 512, big) == ("mfma16", 12)  # K % 8: copies
    ws = lambda M, N, K: mg.migemm_workspace_size(-1, -1, 0, 0, M, N, K, 2, None, K, None, N)
    assert ws(512, 512, 65536) == (mg.OK, 16 * 512 * 512 * 4)
    # 16 tiles of 256x256 in 16 slices of 4096 (the 256x256 tile, configuration 10)
    assert ws(1024, 1024, 65536) == (mg.OK, 16 * 1024 * 1024 * 4)
    # slices of the 256x256 tile would be 512 deep: 4 slices of the 128x128 tile
    assert ws(1024, 1024, 8192) == (mg.OK, 4 * 1024 * 1024 * 4)
    assert ws(128, 128, 4160) == (mg.OK, 0)  # K < 6144
    # configuration 17 asked for: K = 4160 on one tile, 13 slices of 320
    assert mg.migemm_workspace_size(mg.MFMA16, 17, 0, 0, 128, 128, 4160, 2, None, 4160, None,
                                    128) == (mg.OK, 13 * 128 * 128 * 4)
    # slices of the 256x256 tile would be 2048 deep: 2 slices of the 128x128 tile
    assert ws(2048, 1024, 16384) == (mg.OK, 2 * 2048 * 1024 * 4)
    assert ws(2048, 1024, 65536) == (mg.OK, 8 * 2048 * 1024 * 4)
    # more than 128 tiles of 128x128: split-K from K = 12288, and 144 tiles in 2
    # slices would overshoot a round: 36 tiles of 256x256 in 7 slices of 2368
    assert ws(1536, 1536, 8192) == (mg.OK, 0)
    assert _selected(1536, 1536, 8192, 2, 8192, 1536, big) == ("mfma16", 7)
    assert ws(1536, 1536, 16384) == (mg.OK, 7 * 1536 * 1536 * 4)
    # two launches: 16 tiles x 16 slices of the 128x128 kernel, then the sum
    # (4 elements per work-item, 256 work-items per workgroup)
    st, text = mg.migemm_describe_ex(-1, -1, 0, 0, 512, 512, 65536, mg.BF16, None, 65536, None,
                                     512, 0, 512, big)
    d = mg._parse_description(text)
    assert st == mg.OK and d["launches"] == 2 and d["grid0"] == 256 and d["block0"] == 512
    assert d["grid1"] == 512 * 512 // 4 // 256 and d["block1"] == 256
    # K = 8200 on 6 tiles: 15 slices of 576 (the last 136 deep)
    d = mg.describe(mg.MFMA16, 17, 0, 0, 264, 200, 8200, mg.BF16, None, 8200, None, 200, 0, 200,
                    big)
    assert d["launches"] == 2 and d["grid0"] == 6 * 15
    assert d["workspace_bytes"] == 15 * 264 * 200 * 4
    # 16 tiles of 256x256 x 16 slices, 512 threads (the 256x256 tile's 8 waves)
    d = mg.describe(-1, -1, 0, 0, 1024, 1024, 65536, mg.BF16, None, 65536, None, 1024, 0, 1024,
                    big)
    assert d["config"] == 17 and d["grid0"] == 256 and d["block0"] == 512
    # configuration 17 without a workspace: the 128x128 launch alone
    d = mg.describe(mg.MFMA16, 17, 0, 0, 264, 200, 8200, mg.BF16, None, 8200, None, 200, 0, 200,
                    0)
    assert d["launches"] == 1 and d["grid0"] == 6


def test_selection_packs_unaligned_int8():
    """INT8 operands the direct kernel cannot read (K not a multiple of 128, rows
    off 16-byte boundaries) go to the packed configuration 5 once M N K >= 2^27
    and a workspace is lent: each copied operand's rows x K rounded up to 128
    bytes (A' first, rounded up to 256 bytes); an operand already k-contiguous,
    on whole 128-byte lines and with K a multiple of 128 is read in place."""
    big = 1 << 40
    def sel(M, N, K, lda, ldb, ws):
        d = mg.describe(-1, -1, 0, 0, M, N, K, mg.I8, None, lda, None, ldb, mg.I32, N, ws)
        return d["variant"], d["config"]
    assert sel(1000, 1000, 1000, 1000, 1000, big) == ("mfma_i8", 5)
    assert sel(1000, 1000, 1000, 1000, 1000, 0) == ("mfma_i8", 2)       # no workspace
    assert sel(400, 400, 400, 400, 400, big) == ("mfma_i8", 2)          # below 2^27
    assert sel(1024, 1024, 1024, 1024, 1024, big) == ("mfma_i8", 2)     # aligned: in place
    wsz = lambda M, N, K, lda, ldb: mg.migemm_workspace_size(-1, -1, 0, 0, M, N, K, mg.I8, None,
                                                             lda, None, ldb)
    assert wsz(1000, 1000, 1000, 1000, 1000) == (mg.OK, 1024000 + 1000 * 1024)
    assert wsz(3000, 3000, 3072, 3072, 3000) == (mg.OK, 3000 * 3072)     # B' only
    d = mg.describe(-1, -1, 0, 0, 1000, 1000, 1000, mg.I8, None, 1000, None, 1000, mg.I32, 1000,
                    big)
    # the copy (16 x 16 tiles of 64 x 64 for each operand), then the 64x64 tile
    assert d["launches"] == 2 and d["grid0"] == 512 and d["grid1"] == 256


def test_selection_split_k_int8():
    """INT8 products of at most 64 tiles of 256x256 with K >= 8192 and operands the
    direct kernels read run as slices of K (configuration 7) when a workspace
    for their INT32 sums is lent: slices x M x N x 4 bytes, slices of whole
    128-deep k-tiles."""
    def sel(M, N, K, ws):
        d = mg.describe(-1, -1, 0, 0, M, N, K, mg.I8, None, K, None, N, mg.I32, N, ws)
        return d["config"], d["workspace_bytes"], d["launches"]
    big = 1 << 40
    assert sel(1024, 1024, 8192, big) == (7, 16 * 1024 * 1024 * 4, 2)
    assert sel(512, 512, 8192, big) == (7, 16 * 512 * 512 * 4, 2)
    assert sel(2048, 2048, 8192, big) == (7, 4 * 2048 * 2048 * 4, 2)
    assert sel(1024, 1024, 8192, 0)[0] == 4                 # no workspace
    assert sel(1024, 1024, 4096, big)[0] == 2               # K < 8192
    assert sel(2304, 2304, 8192, big)[0] == 4               # 81 tiles
    # K = 8208 (a multiple of 16, not of 128): 13 slices of 640, the last 528 deep
    d = mg.describe(mg.MFMA_I8, 7, 0, 0, 256, 256, 8208, mg.I8, None, 8208, None, 256, mg.I32,
                    256, big)
    assert d["launches"] == 2 and d["grid0"] == 13 and d["workspace_bytes"] == 13 * 256 * 256 * 4


def test_selection_packs_unaligned_fp32():
    """FP32 operands the direct kernel cannot read go to configuration 13 (copies)
    once M N K >= 2^27 and a workspace is lent: each copied operand's rows x K
    rounded up to 32 x 4 bytes, A' first rounded up to 256 bytes."""
    big = 1 << 40
    assert _selected(2049, 2049, 2049, mg.F32, 2049, 2049, big) == ("regtile_mfma", 13)
    assert _selected(2049, 2049, 2049, mg.F32, 2049, 2049, 0) == ("regtile_mfma", 0)
    assert _selected(400, 400, 401, mg.F32, 401, 400, big) == ("regtile_mfma", 2)   # < 2^27
    ws = lambda M, N, K, lda, ldb: mg.migemm_workspace_size(-1, -1, 0, 0, M, N, K, mg.F32, None,
                                                            lda, None, ldb)
    assert ws(2049, 2049, 2049, 2049, 2049) == (mg.OK, 2 * 2049 * 2080 * 4 + 128)
    assert ws(4096, 4096, 4096, 4097, 4097) == (mg.OK, 2 * 4096 * 4096 * 4)


def test_selection_split_k_fp32():
    """FP32 products of at most 128 tiles of 64x64 with K >= 512 run as slices of K
    on the direct 64x64 FP32 tile (configuration 12) when a workspace is lent."""
    big = 1 << 40
    sel = lambda M, N, K: _selected(M, N, K, mg.F32, K, N, big)
    assert sel(512, 512, 512) == ("regtile_mfma", 12)
    assert sel(1024, 512, 1024) == ("regtile_mfma", 12)   # 128 tiles
    assert sel(512, 512, 508) == ("regtile_mfma", 8)      # K < 512
    assert sel(1024, 1024, 4096) == ("regtile_mfma", 8)   # 256 tiles: a full round
    assert mg.migemm_select(512, 512, 4096, mg.F32, None, 4096, None, 512, None, 512) == (
        mg.OK, mg.REGTILE_MFMA, 8)                        # no workspace
    ws = lambda M, N, K: mg.migemm_workspace_size(-1, -1, 0, 0, M, N, K, mg.F32, None, K, None, N)
    assert ws(512, 512, 65536) == (mg.OK, 4 * 512 * 512 * 4)    # 64 tiles, 4 slices
    assert ws(256, 256, 16384) == (mg.OK, 16 * 256 * 256 * 4)   # 16 tiles, 16 slices
    d = mg.describe(-1, -1, 0, 0, 768, 512, 8192, mg.F32, None, 8192, None, 512, 0, 512, big)
    assert d["launches"] == 2 and d["grid0"] == 96 * 2 and d["block0"] == 512


def test_selection_whole_tiles_below_a_round():
    """Whole tiles below one round of 256x256: rounds x time per round (256x256
    21.4, 128x256 13.4, 128x128 9.7 ns per unit of K) picks the tile."""
    sel = lambda M, N: mg.migemm_select(M, N, 4096, mg.BF16, None, 4096, None, N, None, N)[2]
    assert sel(3072, 3072) == 14   # 1 round of 256x256 (144 tiles) against 2 of 128x256
    assert sel(3584, 3584) == 14   # 196 tiles: 1 round against 2 of 128x256, 4 of 128x128
    assert sel(2560, 2560) == 15   # 200 tiles of 128x256: 1 round against 2 of 128x128
    assert sel(2304, 2304) == 15
    assert sel(2048, 2048) == 7    # 256 tiles of 128x128: one round
    assert sel(4096, 4096) == 14   # a round of 256x256 or more: unchanged
    assert sel(1024, 8192) == 15
    assert sel(3000, 3000) == 13   # not whole tiles: unchanged


def test_fp32_selection():
    sel = lambda M, N, K, lda, ldb: mg.migemm_select(M, N, K, mg.F32, None, lda, None, ldb, None, N)
    # direct-staged FP32: 64x64 tiles below a round of 128x128 tiles, 128x128 above
    assert sel(1024, 1024, 1024, 1024, 1024) == (mg.OK, mg.REGTILE_MFMA, 8)
    assert sel(4096, 4096, 4096, 4096, 4096) == (mg.OK, mg.REGTILE_MFMA, 10)
    # 128x128 only where it needs at most half the rounds of the 64x64 tile (two
    # workgroups per CU): 3008^3 is 3 rounds of 128x128 against 5 of 64x64; 2500^3
    # 2 against 3 (after the 4-wide last band is split off); 6000^3 9 against 18
    assert sel(3008, 3008, 3008, 3008, 3008) == (mg.OK, mg.REGTILE_MFMA, 8)
    assert sel(2500, 2500, 2500, 2500, 2500) == (mg.OK, mg.REGTILE_MFMA, 8)
    assert sel(6000, 6000, 6000, 6000, 6000) == (mg.OK, mg.REGTILE_MFMA, 10)
    assert sel(2048, 2048, 2048, 2048, 2048) == (mg.OK, mg.REGTILE_MFMA, 10)
    # K a multiple of 4 (not of the 32-deep k-tile): still direct
    assert sel(1024, 1024, 1000, 1000, 1024) == (mg.OK, mg.REGTILE_MFMA, 8)
    # rows not in whole 16-byte chunks, K not a multiple of 4, N not a multiple of 4:
    # register-staged
    assert sel(1024, 1024, 1024, 1025, 1024) == (mg.OK, mg.REGTILE_MFMA, 2)
    assert sel(1024, 1024, 1001, 1004, 1024) == (mg.OK, mg.REGTILE_MFMA, 2)
    assert sel(4096, 4094, 4096, 4096, 4094) == (mg.OK, mg.REGTILE_MFMA, 0)
    for c in (8, 9, 10, 11):
        assert mg.migemm_config_name(mg.REGTILE_MFMA, c).startswith("direct")


def test_workspace_size():
    ws = lambda *a: mg.migemm_workspace_size(*a)
    # 2050 x 2047 x 2056 FP16, ldb = 2047: both copied as k-contiguous images with
    # rows on 128-byte lines (leading dimension 2112): A' (2050 x 2112, A's rows of
    # 4112 bytes straddle lines; rounded up to 256 bytes) then B' (2047 x 2112)
    c3r = (2050 * 2112 * 2 + 255) // 256 * 256 + 2047 * 2112 * 2
    assert c3r == 17305728
    assert ws(-1, -1, 0, 0, 2050, 2047, 2056, 1, None, 2056, None, 2047) == (mg.OK, c3r)
    # K = 2052 (not a multiple of 8) and operands given transposed (A stored K x M
    # with an odd leading dimension, B stored N x K): the same copies
    assert ws(-1, -1, 0, 0, 2050, 2047, 2052, 1, None, 2052, None, 2047) == (mg.OK, c3r)
    assert ws(-1, -1, 1, 1, 2050, 2047, 2052, 1, None, 2051, None, 2052) == (mg.OK, c3r)
    # A on 128-byte lines (lda 2112), B's rows aligned but N = 2047: only B copied
    assert ws(-1, -1, 0, 0, 2050, 2047, 2056, 1, None, 2112, None, 2048) == \
        (mg.OK, 2047 * 2112 * 2)
    # K a multiple of 64 and A aligned: only B is copied
    assert ws(-1, -1, 0, 0, 4096, 4096, 4096, 2, None, 4096, None, 4097) == (mg.OK, 4096 * 4096 * 2)
    # aligned, FP32, INT8, small, empty: none
    # FP32 with A's rows not in whole 16-byte chunks: A copied, K rounded up to 32
    assert ws(-1, -1, 0, 0, 1024, 1024, 1024, 0, None, 1025, None, 1024) == \
        (mg.OK, 1024 * 1024 * 4)
    for a in [(8192, 8192, 8192, 2, 8192, 8192), (1024, 1024, 1024, 0, 1024, 1024),
              (8192, 8192, 8192, 3, 8192, 8192), (100, 100, 100, 1, 101, 100),
              (0, 4096, 4096, 1, 4097, 4096), (4096, 4096, 0, 1, 1, 4097)]:
        M, N, K, dt, lda, ldb = a
        assert ws(-1, -1, 0, 0, M, N, K, dt, None, lda, None, ldb) == (mg.OK, 0), a
    # a forced packed configuration reports its copies; any other forced one none
    assert ws(mg.MFMA16, 12, 0, 0, 512, 512, 100, 1, None, 100, None, 512)[1] == 512 * 128 * 2
    assert ws(mg.MFMA16, 12, 0, 0, 512, 512, 200, 1, None, 200, None, 512)[1] == 512 * 256 * 2
    assert ws(mg.MFMA16, 12, 0, 0, 512, 512, 192, 1, None, 192, None, 512)[1] == 0
    assert ws(mg.MFMA16, 2, 0, 0, 2050, 2047, 2056, 1, None, 2056, None, 2047) == (mg.OK, 0)
    # argument errors as for the product
    assert ws(-1, -1, 0, 0, -1, 4, 4, 1, None, 4, None, 4)[0] == mg.ERR_INVALID_ARG
    assert mg.lib().migemm_workspace_size(-1, -1, 0, 0, 4, 4, 4, 1, None, 4, None, 4,
                                          None) == mg.ERR_INVALID_ARG


def test_describe_split_bands():
    """A last band of tile rows or columns that would start a second round of
    workgroups runs as launches of its own after the whole tiles: up to 16 rows
    on the skinny kernel (16 columns of C per workgroup, sixteen waves), up to 16
    columns on the skinny kernel as the transposed product (16 rows of C per
    workgroup; eight waves when B is row-major), wider tails on the 64x64 tile;
    FP16/BF16 and FP32 alike."""
    def launches(M, N, K, cfg=-1, dt=mg.BF16):
        d = mg.describe(-1 if cfg < 0 else mg.MFMA16, cfg, 0, 0, M, N, K, dt, None, K,
                        None, N, 0, N, 0)
        return d["config"], [(d[f"grid{i}"], d[f"block{i}"]) for i in range(d["launches"])]
    # 256x256 tiles; whole tiles on the ping-pong kernel (8 waves, 512 work-items)
    assert launches(4100, 4096, 4096) == (10, [(256, 512), (256, 1024)])
    assert launches(4096, 4104, 4096) == (10, [(256, 512), (256, 512)])
    assert launches(4100, 4104, 4096) == (10, [(256, 512), (257, 1024), (256, 512)])
    assert launches(8192, 8200, 8192) == (10, [(1024, 512), (512, 512)])
    # wider tails: one band of 64x64 tiles
    assert launches(4160, 4096, 4096) == (10, [(256, 512), (64, 512)])
    assert launches(4096, 4160, 4096) == (10, [(256, 512), (64, 512)])
    # 128x128 tiles: eight tail columns
    assert launches(2048, 2056, 2048) == (7, [(256, 512), (128, 512)])
    # no split where the whole tiles alone would not save a round
    assert launches(3080, 3072, 3072) == (13, [(300, 512)])
    assert launches(4352, 4096, 4096) == (14, [(272, 512)])
    assert launches(4096, 4096, 4096) == (14, [(256, 512)])
    # FP32 on its matrix-core kernels: the 128x128 tile (configuration 10) and the
    # 64x64 one (8) with tails of up to 16 on the FP32 skinny kernel; a wider
    # tail of the 64x64 tile is left in place (it would cost the same round)
    F32 = mg.F32
    assert launches(2056, 2048, 2048, dt=F32) == (10, [(256, 512), (128, 1024)])
    assert launches(2048, 2056, 2048, dt=F32) == (10, [(256, 512), (128, 512)])
    assert launches(2100, 2048, 2048, dt=F32) == (10, [(256, 512), (32, 512)])
    assert launches(1032, 1024, 1024, dt=F32) == (8, [(256, 512), (64, 1024)])
    assert launches(1080, 1024, 1024, dt=F32) == (8, [(272, 512)])
    # INT8: whole 256x256 tiles on the direct ping-pong kernel whenever the
    # operands suit it, the rest after them (the skinny kernel up to 16, also
    # for a tail that ends inside a 16-byte chunk; the register-staged 64x64
    # tile beyond)
    def launches_i8(M, N, K, ldb):
        d = mg.describe(-1, -1, 0, 0, M, N, K, mg.I8, None, K, None, ldb, mg.I32, N, 0)
        return d["config"], [(d[f"grid{i}"], d[f"block{i}"]) for i in range(d["launches"])]
    assert launches_i8(8192, 8192, 8192, 8192) == (4, [(1024, 512)])
    assert launches_i8(8200, 8192, 8192, 8192) == (3, [(1024, 512), (512, 1024)])
    assert launches_i8(8192, 8208, 8192, 8208) == (3, [(1024, 512), (512, 512)])
    assert launches_i8(8192, 8200, 8192, 8208) == (3, [(1024, 512), (512, 512)])
    assert launches_i8(8400, 8192, 8192, 8192) == (3, [(1024, 512), (512, 256)])
    # below a round of 256x256 tiles too, once the product is large (M N K >= 5e9)
    # or K long: 64 whole tiles on the direct kernel, then 8 rows on the skinny one
    assert launches_i8(2056, 2048, 2048, 2048) == (3, [(64, 512), (128, 1024)])
    assert launches_i8(3072, 3072, 3072, 3072) == (4, [(144, 512)])
    assert launches_i8(512, 512, 8192, 512) == (4, [(4, 512)])
    # smaller: the register-staged 64x64 tile (4 waves), also for K not a
    # multiple of 128
    assert launches_i8(1536, 1536, 1536, 1536) == (2, [(576, 256)])
    assert launches_i8(1024, 1024, 4096, 1024) == (2, [(256, 256)])
    assert launches_i8(3072, 3072, 3080, 3072)[0] == 1


def test_describe():
    st, text = mg.migemm_describe(8192, 8192, 8192, mg.BF16, 8192, 8192, 8192)
    assert st == mg.OK
    d = mg._parse_description(text)
    assert d["variant"] == "mfma16" and d["config"] == 14
    assert d["config_name"] == mg.migemm_config_name(mg.MFMA16, 14)
    assert d["workspace_bytes"] == 0 and d["launches"] == 1
    assert d["grid0"] == 1024 and d["block0"] == 512
    # on a machine with a GPU the kernel's attributes follow; without one, a note
    assert "regs0" in d or "resources0" in d
    # the ragged product with a workspace: the copies (33 x 33 tiles of 64 x 64 for
    # A', 32 x 33 for B'), then 256 tiles of 128 x 128 over rows 0..2047, then the
    # last 2 rows on 128 workgroups of 16 columns
    st, text = mg.migemm_describe_ex(-1, -1, 0, 0, 2050, 2047, 2056, mg.F16, None, 2056, None,
                                     2047, mg.F32, 2047, 1 << 30)
    d = mg._parse_description(text)
    assert st == mg.OK and d["config"] == 12 and d["workspace_bytes"] == 17305728
    assert d["launches"] == 3 and d["grid0"] == 33 * 33 + 32 * 33 and d["grid1"] == 256
    assert d["grid2"] == 128 and d["block2"] == 1024
    assert d["workspace_lent"] == 1 << 30
    # K a multiple of 8 but not of 64: configuration 7 runs its own direct kernel
    # (8 waves); K not a multiple of 8: the register-staged 128x128 one (4 waves)
    d = mg.describe(mg.MFMA16, 7, 0, 0, 300, 264, 72, mg.BF16, None, 72, None, 264, 0, 264, 0)
    assert d["launches"] == 1 and d["grid0"] == 9 and d["block0"] == 512
    d = mg.describe(mg.MFMA16, 7, 0, 0, 300, 264, 68, mg.BF16, None, 72, None, 264, 0, 264, 0)
    assert d["launches"] == 1 and d["grid0"] == 9 and d["block0"] == 256
    # FP32 and INT8
    d = mg._parse_description(mg.migemm_describe(1024, 1024, 1024, mg.F32, 1024, 1024, 1024)[1])
    assert d["variant"] == "regtile_mfma" and d["launches"] == 1
    d = mg._parse_description(mg.migemm_describe(8192, 8192, 8192, mg.I8, 8192, 8192, 8192)[1])
    assert d["variant"] == "mfma_i8" and d["config"] == 4
    # K == 0 launches the empty product, M == 0 nothing
    assert mg._parse_description(mg.migemm_describe(64, 64, 0, 0, 1, 64, 64)[1])["launches"] == 1
    assert mg._parse_description(mg.migemm_describe(0, 64, 64, 0, 64, 64, 64)[1])["launches"] == 0
    # a buffer too small: cut short, status says so; bad arguments: no text
    st, text = mg.migemm_describe(8192, 8192, 8192, mg.BF16, 8192, 8192, 8192, buflen=20)
    assert st == mg.ERR_INVALID_ARG and len(text) == 19
    assert mg.migemm_describe(8, 8, 8, 9, 8, 8, 8)[0] == mg.ERR_INVALID_ARG
    assert mg.lib().migemm_describe(8, 8, 8, 0, 8, 8, 8, None, 10) == mg.ERR_INVALID_ARG


def test_gemm_ws_argument_checks():
    a = (-1, -1, 0, 0, 8, 5, 4, 1, P, 4, 2 * P, 5, 1.0, 0.0, 0, 3 * P, 5)
    assert mg.migemm_gemm_ws(*a, None, -1, None) == mg.ERR_INVALID_ARG
    bad = list(a)
    bad[4] = -1
    assert mg.migemm_gemm_ws(*bad, None, 0, None) == mg.ERR_INVALID_ARG
    assert mg.migemm_gemm_ws(mg.LDS_TILED, -1, *a[2:], None, 0, None) == mg.ERR_UNSUPPORTED


class _FakeCudaTensor:
    """Enough of a torch tensor on cuda:0 for gemm()'s argument checks, on a
    machine without a GPU (never dereferenced: the checks fail first)."""

    def __init__(self, rows, cols):
        import torch
        self.device = torch.device("cuda", 0)
        self.dtype = torch.float32
        self.shape = (rows, cols)

    def stride(self, d=None):
        s = (self.shape[1], 1)
        return s if d is None else s[d]

    def dim(self):
        return 2

    def data_ptr(self):
        return P


def test_gemm_rejects_output_on_another_device():
    import torch
    a, b = _FakeCudaTensor(8, 4), _FakeCudaTensor(4, 5)
    with pytest.raises(ValueError, match="out must be on the GPU"):
        mg.gemm(a, b, out=torch.empty((8, 5)))
    with pytest.raises(ValueError, match="b must be on the GPU"):
        mg.gemm(a, torch.empty((4, 5)))
    other = _FakeCudaTensor(8, 5)
    other.device = torch.device("cuda", 1)
    with pytest.raises(ValueError, match="out is on cuda:1"):
        mg.gemm(a, b, out=other)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(mg, "_lib", None)
    monkeypatch.setattr(mg, "LIBRARY_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mg.migemm_variant_count()
