"""Helpers for the GPU parity tests: run the library through its C ABI on
seeded inputs and compare element by element with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import dense_gemm_16_amd as mg
import oracle
from oracle.check import compare, tolerance
from dense_gemm_16_amd import inputs

DT_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def say(msg: str):
    """Name the case before a GPU step, flushed, so a fault report can be attributed."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_device_with_ld(x: torch.Tensor, ld: int | None = None, offset: int = 0):
    """Copy a CPU matrix to the GPU inside a larger buffer: row stride ``ld`` and a start
    ``offset`` elements into the allocation (offset 1 makes the base misaligned)."""
    rows, cols = x.shape
    ld = ld or max(cols, 1)
    buf = torch.full((offset + max(rows, 1) * ld + 8,), float("nan"), dtype=x.dtype,
                     device="cuda")
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols] if rows else \
        buf[offset:offset].view(0, cols)
    view.copy_(x.to("cuda"))
    return view, buf


def lend_workspace(variant, config, op_a, op_b, M, N, K, dt, pa, lda, pb, ldb, ws):
    """(pointer, bytes, tensor) of the workspace a test lends: ws == "auto" lends
    what migemm_workspace_size asks for (None when it asks for none), None lends
    nothing, an int lends that many bytes."""
    if ws is None:
        return None, 0, None
    if ws == "auto":
        st, n = mg.migemm_workspace_size(variant, config, op_a, op_b, M, N, K, dt, pa, lda, pb,
                                         ldb)
        assert st == mg.OK
    else:
        n = int(ws)
    if n == 0:
        return None, 0, None
    t = torch.empty(n, dtype=torch.uint8, device="cuda")
    return t.data_ptr(), n, t


def run_gemm(A: torch.Tensor, B: torch.Tensor, dtype: str, variant=-1, config=-1, lda=None,
             ldb=None, ldc=None, a_off=0, b_off=0, c_off=0, poison=True, ws="auto"):
    """Run C = A x B through migemm_gemm_ws, lending the workspace the call asks
    for (ws="auto"; ws=None lends none, as migemm_gemm_variant does); returns (C
    on CPU as float32, C buffer)."""
    M, K = A.shape
    N = B.shape[1]
    dA, _ = to_device_with_ld(A, lda, a_off)
    dB, _ = to_device_with_ld(B, ldb, b_off)
    ldc = ldc or max(N, 1)
    cbuf = torch.full((c_off + max(M, 1) * ldc + 64,), float("nan") if poison else 0.0,
                      dtype=torch.float32, device="cuda")
    dC = cbuf[c_off:c_off + M * ldc].view(M, ldc)[:, :N] if M else cbuf[:0].view(0, N)
    stream = torch.cuda.current_stream().cuda_stream
    pa = dA.data_ptr() if dA.numel() else None
    pb = dB.data_ptr() if dB.numel() else None
    lda, ldb = lda or max(K, 1), ldb or max(N, 1)
    wp, wn, _wt = lend_workspace(variant, config, 0, 0, M, N, K, DT_CODE[dtype], pa, lda, pb,
                                 ldb, ws)
    if wp is None:
        st = mg.migemm_gemm_variant(variant, config, M, N, K, DT_CODE[dtype], pa, lda, pb, ldb,
                                    dC.data_ptr() if dC.numel() else None, ldc, stream)
    else:
        st = mg.migemm_gemm_ws(variant, config, 0, 0, M, N, K, DT_CODE[dtype], pa, lda, pb, ldb,
                               1.0, 0.0, 0, dC.data_ptr() if dC.numel() else None, ldc, wp, wn,
                               stream)
    torch.cuda.synchronize()
    assert st == mg.OK, f"status {st}: {mg.migemm_status_string(st)} hip={mg.migemm_last_hip_error()}"
    return dC.cpu().clone(), cbuf


def oracle_ref(A: torch.Tensor, B: torch.Tensor, dtype: str):
    return oracle.gemm(inputs.to_bits(A), inputs.to_bits(B), DT_CODE[dtype])


def check(Cgpu: torch.Tensor, A, B, dtype: str, exact=False, ref=None):
    C, S = ref if ref is not None else oracle_ref(A, B, dtype)
    r = compare(Cgpu.numpy(), C, S, tol=None if exact else tolerance(DT_CODE[dtype]), exact=exact)
    assert r.ok, str(r)
    return r


def sampled_entries(M, N, n, seed=0, include_edges=True):
    """Sampled (row, col) pairs: random plus the four corners and last row/col."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, n))
    cols = list(rng.integers(0, N, n))
    if include_edges:
        for r, c in [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]:
            rows.append(r)
            cols.append(c)
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


TORCH_OF = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}


def run_gemm_ex(A: torch.Tensor, B: torch.Tensor, dtype: str, alpha: float, beta: float,
                c_code: int, c_old: torch.Tensor | None = None, variant=-1, config=-1,
                ldc=None, c_off=0, ta=False, tb=False, lda=None, ldb=None, a_off=0, b_off=0,
                ws="auto"):
    """C = alpha * A x B + beta * C_old through migemm_gemm_ws (lending the
    workspace as run_gemm does; without one, migemm_gemm_ex_variant), C stored as
    c_code (0 FP32, 1 FP16, 2 BF16).  A (M x K) and B (K x N) are the operands of
    the product; with ta / tb they are stored transposed (K x M, N x K) on the GPU
    and passed with MIGEMM_OP_T.  Operands and C sit inside NaN-filled buffers
    (row strides lda, ldb, ldc; offsets in elements); with beta == 0 the C window
    starts as NaN too, so a read of the previous C would show.  Returns (C on the
    CPU in its own dtype, C buffer, the window's mask in the buffer)."""
    M, K = A.shape
    N = B.shape[1]
    sA = A.t().contiguous() if ta else A
    sB = B.t().contiguous() if tb else B
    dA, _ = to_device_with_ld(sA, lda, a_off)
    dB, _ = to_device_with_ld(sB, ldb, b_off)
    lda = lda or max(sA.shape[1], 1)
    ldb = ldb or max(sB.shape[1], 1)
    ldc = ldc or max(N, 1)
    tdt = TORCH_OF[c_code]
    cbuf = torch.full((c_off + max(M, 1) * ldc + 64,), float("nan"), dtype=tdt, device="cuda")
    dC = cbuf[c_off:c_off + M * ldc].view(M, ldc)[:, :N] if M else cbuf[:0].view(0, N)
    if beta != 0.0:
        assert c_old is not None and c_old.dtype == tdt
        dC.copy_(c_old.to("cuda"))
    mask = torch.zeros(cbuf.shape, dtype=torch.bool)
    if M:
        mask[c_off:c_off + M * ldc].view(M, ldc)[:, :N] = True
    stream = torch.cuda.current_stream().cuda_stream
    pa = dA.data_ptr() if dA.numel() else None
    pb = dB.data_ptr() if dB.numel() else None
    pc = dC.data_ptr() if dC.numel() else None
    wp, wn, _wt = lend_workspace(variant, config, int(ta), int(tb), M, N, K, DT_CODE[dtype], pa,
                                 lda, pb, ldb, ws)
    if wp is None:
        st = mg.migemm_gemm_ex_variant(variant, config, int(ta), int(tb), M, N, K,
                                       DT_CODE[dtype], pa, lda, pb, ldb, alpha, beta, c_code, pc,
                                       ldc, stream)
    else:
        st = mg.migemm_gemm_ws(variant, config, int(ta), int(tb), M, N, K, DT_CODE[dtype], pa,
                               lda, pb, ldb, alpha, beta, c_code, pc, ldc, wp, wn, stream)
    torch.cuda.synchronize()
    assert st == mg.OK, f"status {st}: {mg.migemm_status_string(st)} hip={mg.migemm_last_hip_error()}"
    return dC.cpu().clone(), cbuf.cpu(), mask


def check_ex(Cgpu: torch.Tensor, A, B, dtype: str, alpha, beta, c_code, c_old=None, ref=None,
             exact=False):
    """Compare a general-form result with the oracle's update (tolerance plus the final
    rounding of the output format, or exact)."""
    acc, S = ref if ref is not None else oracle_ref(A, B, dtype)
    old = inputs.to_bits(c_old) if (c_old is not None and beta != 0.0) else None
    want, scale = oracle.epilogue(acc, S, alpha, beta, c_code, old)
    got = Cgpu.double().numpy()
    r = compare(got, want, scale, tol=None if exact else tolerance(DT_CODE[dtype]), exact=exact,
                out_dtype=None if exact else c_code)
    assert r.ok, str(r)
    return r


def padding_untouched(cbuf: torch.Tensor, mask: torch.Tensor) -> bool:
    return bool(torch.isnan(cbuf[~mask].float()).all())
