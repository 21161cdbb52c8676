"""Calls captured into a HIP graph (torch.cuda.CUDAGraph on a side stream) and
replayed: the library only launches kernels on the caller's stream (no
allocation, no host wait, no memset), so a captured call must produce, on every
replay, exactly what the same call produces eagerly, also where a call is two
launches sharing a workspace (copies then the product, slices then their
sum).  Between replays C is
reset (to its previous value for an update, else poisoned) by eager work on the
stream and the program synchronises; each replay's C is compared bit for bit
with the eager result.  Cases: a plain FP16 product,
the packed path with its copy launch and workspace, a split product (whole
tiles, then the skinny tail), FP32 (in place, in slices of K, and copied),
INT8, and the general output step with
beta != 0 into BF16 C (so a replay that reads a stale C would show).
"""
import pytest
import torch

import dense_gemm_16_amd as mg
from dense_gemm_16_amd import inputs
from gpu_helpers import say

pytestmark = pytest.mark.gpu

TORCH_C = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16, 4: torch.int32}


def _case(M, N, K, dtype, alpha=1.0, beta=0.0, c_code=None, ldb=None):
    dist = "uniform" if dtype == "i8" else "normal"
    A, B = inputs.pair(M, N, K, dtype, dist, seed=M + 2 * N + 3 * K)
    code = inputs.DTYPE_CODES[dtype]
    c_code = (4 if dtype == "i8" else 0) if c_code is None else c_code
    dA = A.cuda()
    ldb = ldb or N
    dB = torch.zeros((K, ldb), dtype=B.dtype, device="cuda")
    dB[:, :N] = B.cuda()
    C0 = (torch.rand((M, N), generator=torch.Generator().manual_seed(K)) - 0.5).to(TORCH_C[c_code])
    C0 = C0.cuda()
    C = torch.empty_like(C0)
    st, nws = mg.migemm_workspace_size(-1, -1, 0, 0, M, N, K, code, dA.data_ptr(), K,
                                       dB.data_ptr(), ldb)
    assert st == mg.OK
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")

    def call(stream_ptr):
        st = mg.migemm_gemm_ws(-1, -1, 0, 0, M, N, K, code, dA.data_ptr(), K, dB.data_ptr(), ldb,
                               alpha, beta, c_code, C.data_ptr(), N, ws.data_ptr() if nws else None,
                               nws, stream_ptr)
        assert st == mg.OK, mg.migemm_status_string(st)

    return C, C0, call


@pytest.mark.parametrize("M,N,K,dtype,alpha,beta,c_code,ldb", [
    (256, 256, 256, "f16", 1.0, 0.0, None, None),
    (2050, 2047, 2056, "f16", 1.0, 0.0, None, 2047),   # copies, 128x128 product, skinny tail
    (4100, 4096, 128, "bf16", 1.0, 0.0, None, None),   # whole tiles, then the skinny tail
    (1024, 1024, 1024, "f32", 1.0, 0.0, None, None),
    (512, 512, 512, "i8", 1.0, 0.0, None, None),
    (1000, 1032, 520, "bf16", 0.5, -1.25, 2, None),    # general output step, beta != 0
    (512, 512, 16384, "bf16", 1.0, 0.0, None, None),   # split-K: slices, then their sum
    (512, 384, 8192, "f16", -0.5, 0.75, 1, None),      # split-K with the general output step
    (512, 512, 4096, "f32", 1.0, 0.0, None, None),     # FP32 split-K
    (1000, 1000, 1000, "i8", 1.0, 0.0, None, None),    # INT8 copies, then the 64x64 tile
    (512, 512, 8192, "i8", 1.0, 0.0, None, None),      # INT8 split-K
    (1023, 1023, 1023, "f32", 1.0, 0.0, None, None),   # FP32 copies, then the 64x64 tile
    (2049, 2049, 2049, "f32", 0.5, -1.0, 2, None),     # FP32 copies, 128x128, general output
])
def test_graph_replays_match_eager(M, N, K, dtype, alpha, beta, c_code, ldb):
    say(f"graph {M}x{N}x{K} {dtype} alpha={alpha} beta={beta} c_code={c_code} ldb={ldb}")
    C, C0, call = _case(M, N, K, dtype, alpha, beta, c_code, ldb)
    # eager
    C.copy_(C0)
    call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = C.clone()
    # capture one call on a side stream (default priority)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for r in range(3):
        # eager work between replays: C back to C0 for the update (beta != 0),
        # else poisoned, so that an element a replay does not write would show
        if beta != 0.0:
            C.copy_(C0)
        else:
            C.fill_(float("nan") if C.is_floating_point() else -2147483641)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, want), f"replay {r} differs from the eager call"
    del g
