"""migemm_gemm_noalloc, the entry point that allocates nothing, against
migemm_gemm_ws (the entry point it is a variant of) lent a torch workspace, and
both against the oracle.

Two calls in a row on the packed path (ragged K, odd leading dimension of B),
the second on a smaller product: it reuses the scratch array the first call
filled, so any stale byte it read would show; the same for split-K, whose
slices' sums sit in the array.  Then a product that needs no
scratch, and one that needs more than the array holds (rejected before any
launch).
"""
import pytest
import torch

import dense_gemm_16_amd as mg
from dense_gemm_16_amd import inputs
from gpu_helpers import DT_CODE, check_ex, say, to_device_with_ld

pytestmark = pytest.mark.gpu


def _both(M, N, K, dtype, ldb, seed):
    A, B = inputs.pair(M, N, K, dtype, "normal", seed=seed)
    dA, _ = to_device_with_ld(A, K, 0)
    dB, _ = to_device_with_ld(B, ldb, 0)
    dt = DT_CODE[dtype]
    st, need = mg.migemm_workspace_size(-1, -1, 0, 0, M, N, K, dt, dA.data_ptr(), K,
                                        dB.data_ptr(), ldb)
    assert st == mg.OK
    stream = torch.cuda.current_stream().cuda_stream
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    C_ws = torch.full((M, N), float("nan"), device="cuda")
    C_na = torch.full((M, N), float("nan"), device="cuda")
    say(f"noalloc {dtype} {M}x{N}x{K} ldb={ldb}: workspace entry point ({need} bytes lent)")
    st = mg.migemm_gemm_ws(-1, -1, 0, 0, M, N, K, dt, dA.data_ptr(), K, dB.data_ptr(), ldb,
                           1.0, 0.0, 0, C_ws.data_ptr(), N, ws.data_ptr(), need, stream)
    assert st == mg.OK
    say(f"noalloc {dtype} {M}x{N}x{K} ldb={ldb}: allocation-free entry point")
    st = mg.migemm_gemm_noalloc(-1, -1, 0, 0, M, N, K, dt, dA.data_ptr(), K, dB.data_ptr(), ldb,
                                1.0, 0.0, 0, C_na.data_ptr(), N, stream)
    assert st == mg.OK, mg.migemm_status_string(st)
    torch.cuda.synchronize()
    return A, B, need, C_ws.cpu(), C_na.cpu()


def test_noalloc_matches_workspace_entry_point_twice():
    first = None
    for (M, N, K, dtype, seed) in [(1030, 1023, 1032, "f16", 5), (600, 517, 520, "bf16", 6)]:
        A, B, need, C_ws, C_na = _both(M, N, K, dtype, N, seed)
        assert 0 < need <= mg.NOALLOC_SCRATCH_BYTES
        if first is not None:
            assert need < first, "the second product is the smaller one"
        first = need
        # same selection, same kernels, same summation order: identical bits
        assert torch.equal(C_ws.view(torch.int32), C_na.view(torch.int32))
        check_ex(C_na, A, B, dtype, 1.0, 0.0, 0, None)


def test_noalloc_split_k_twice():
    """Split-K keeps its slices' sums in the scratch array: two long products in a
    row, the second smaller, each matching the workspace entry point bit for bit."""
    first = None
    for (M, N, K, dtype, seed) in [(512, 512, 16384, "bf16", 8), (264, 200, 8200, "f16", 9)]:
        st, text = mg.migemm_describe_ex(-1, -1, 0, 0, M, N, K, DT_CODE[dtype], None, K, None, N,
                                         0, N, mg.NOALLOC_SCRATCH_BYTES)
        assert st == mg.OK and mg._parse_description(text)["config"] == 17
        A, B, need, C_ws, C_na = _both(M, N, K, dtype, N, seed)
        assert 0 < need <= mg.NOALLOC_SCRATCH_BYTES
        if first is not None:
            assert need < first, "the second product is the smaller one"
        first = need
        assert torch.equal(C_ws.view(torch.int32), C_na.view(torch.int32))
        check_ex(C_na, A, B, dtype, 1.0, 0.0, 0, None)


def test_noalloc_fp32_copies_twice():
    """FP32 operands the direct kernel cannot read are copied into the scratch
    array: 2049^3, then the smaller 1023^3, each matching the workspace entry
    point bit for bit."""
    first = None
    for (M, N, K, seed) in [(2049, 2049, 2049, 10), (1023, 1023, 1023, 11)]:
        st, text = mg.migemm_describe_ex(-1, -1, 0, 0, M, N, K, mg.F32, None, K, None, N,
                                         0, N, mg.NOALLOC_SCRATCH_BYTES)
        assert st == mg.OK and mg._parse_description(text)["config"] == 13
        A, B, need, C_ws, C_na = _both(M, N, K, "f32", N, seed)
        assert 0 < need <= mg.NOALLOC_SCRATCH_BYTES
        if first is not None:
            assert need < first, "the second product is the smaller one"
        first = need
        assert torch.equal(C_ws.view(torch.int32), C_na.view(torch.int32))
        check_ex(C_na, A, B, "f32", 1.0, 0.0, 0, None)


def test_noalloc_without_scratch_need():
    A, B, need, C_ws, C_na = _both(512, 512, 512, "bf16", 512, 7)
    assert need == 0
    assert torch.equal(C_ws.view(torch.int32), C_na.view(torch.int32))
    check_ex(C_na, A, B, "bf16", 1.0, 0.0, 0, None)


def test_noalloc_rejects_products_beyond_its_scratch():
    # 4100 x 4100 x 4100 FP16 with an odd ldb packs both operands: 68,224,000 bytes
    M = N = K = 4100
    st, need = mg.migemm_workspace_size(-1, -1, 0, 0, M, N, K, 1, None, K, None, N + 1)
    assert st == mg.OK and need > mg.NOALLOC_SCRATCH_BYTES
    say("noalloc oversized product: rejected before any launch")
    st = mg.migemm_gemm_noalloc(-1, -1, 0, 0, M, N, K, 1, 1 << 20, K, 1 << 40, N + 1, 1.0, 0.0,
                                0, 1 << 44, N, None)
    assert st == mg.ERR_WORKSPACE
