"""Python binding of libmigemm (the gfx950 dense matrix-multiply library).

Argument marshalling only: every step of the product runs in the library's HIP
kernels.  The functions named ``migemm_*`` mirror the C ABI in
``include/migemm.h`` one for one (integers and raw device pointers);
``gemm`` is a convenience wrapper over torch tensors that derives the sizes,
leading dimensions, pointers and the current stream, lends the workspace that
``migemm_workspace_size`` asks for (a torch allocation on the same stream) and
calls ``migemm_gemm_ws``.

The library is loaded on first use from this package's directory.  If it has
not been built, every call raises ``RuntimeError``: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libmigemm.so")

F32, F16, BF16, I8, I32 = 0, 1, 2, 3, 4
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 64 << 20  # the allocation-free entry point's scratch per GPU
OP_N, OP_T = 0, 1
VARIANT_AUTO, NAIVE, LDS_TILED, REGTILE_VALU, REGTILE_MFMA, MFMA16, MFMA_I8 = -1, 0, 1, 2, 3, 4, 5

# Every symbol the header declares (checked by the CPU test suite).
EXPORTS = ("migemm_gemm", "migemm_gemm_variant", "migemm_gemm_ex", "migemm_gemm_ex_variant",
           "migemm_gemm_ws", "migemm_gemm_noalloc", "migemm_workspace_size", "migemm_describe",
           "migemm_describe_ex",
           "migemm_convert",
           "migemm_variant_count", "migemm_variant_name",
           "migemm_variant_supports", "migemm_config_count", "migemm_config_name",
           "migemm_select", "migemm_status_string", "migemm_last_hip_error", "migemm_version")

_lib = None


class MigemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = migemm_status_string(status)
        if status == ERR_HIP:
            msg += f" (hipError_t {migemm_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def lib():
    """The loaded library (ctypes.CDLL); raises RuntimeError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise RuntimeError(f"libmigemm.so is not built ({LIBRARY_PATH}); run "
                           "`python dense_gemm_16_amd/build.py` or __graft_entry__.build()")
    L = ctypes.CDLL(LIBRARY_PATH)
    i64, i32, vp, cp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_char_p
    L.migemm_gemm.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, vp, i64, vp]
    L.migemm_gemm.restype = i32
    L.migemm_gemm_variant.argtypes = [i32, i32, i64, i64, i64, i32, vp, i64, vp, i64, vp, i64, vp]
    L.migemm_gemm_variant.restype = i32
    f32 = ctypes.c_float
    L.migemm_gemm_ex.argtypes = [i32, i32, i64, i64, i64, i32, vp, i64, vp, i64, f32, f32, i32,
                                 vp, i64, vp]
    L.migemm_gemm_ex.restype = i32
    L.migemm_gemm_ex_variant.argtypes = [i32, i32, i32, i32, i64, i64, i64, i32, vp, i64, vp, i64,
                                         f32, f32, i32, vp, i64, vp]
    L.migemm_gemm_ex_variant.restype = i32
    L.migemm_gemm_ws.argtypes = [i32, i32, i32, i32, i64, i64, i64, i32, vp, i64, vp, i64,
                                 f32, f32, i32, vp, i64, vp, i64, vp]
    L.migemm_gemm_ws.restype = i32
    L.migemm_gemm_noalloc.argtypes = [i32, i32, i32, i32, i64, i64, i64, i32, vp, i64, vp, i64,
                                      f32, f32, i32, vp, i64, vp]
    L.migemm_gemm_noalloc.restype = i32
    L.migemm_workspace_size.argtypes = [i32, i32, i32, i32, i64, i64, i64, i32, vp, i64, vp,
                                        i64, ctypes.POINTER(i64)]
    L.migemm_workspace_size.restype = i32
    L.migemm_describe.argtypes = [i64, i64, i64, i32, i64, i64, i64, cp, i32]
    L.migemm_describe.restype = i32
    L.migemm_describe_ex.argtypes = [i32, i32, i32, i32, i64, i64, i64, i32, vp, i64, vp, i64,
                                     i32, i64, i64, cp, i32]
    L.migemm_describe_ex.restype = i32
    L.migemm_convert.argtypes = [i32, i32, i64, i64, vp, i64, vp, i64, vp]
    L.migemm_convert.restype = i32
    L.migemm_variant_count.argtypes = []
    L.migemm_variant_count.restype = i32
    L.migemm_variant_name.argtypes = [i32]
    L.migemm_variant_name.restype = cp
    L.migemm_variant_supports.argtypes = [i32, i32]
    L.migemm_variant_supports.restype = i32
    L.migemm_config_count.argtypes = [i32]
    L.migemm_config_count.restype = i32
    L.migemm_config_name.argtypes = [i32, i32]
    L.migemm_config_name.restype = cp
    L.migemm_select.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, vp, i64,
                                ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.migemm_select.restype = i32
    L.migemm_status_string.argtypes = [i32]
    L.migemm_status_string.restype = cp
    L.migemm_last_hip_error.argtypes = []
    L.migemm_last_hip_error.restype = i32
    L.migemm_version.argtypes = []
    L.migemm_version.restype = i32
    _lib = L
    return L


# ---------------------------------------------------------------- C ABI mirror

def migemm_gemm(M, N, K, dtype, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return lib().migemm_gemm(M, N, K, dtype, A, lda, B, ldb, C, ldc, stream)


def migemm_gemm_variant(variant, config, M, N, K, dtype, A, lda, B, ldb, C, ldc,
                        stream=None) -> int:
    return lib().migemm_gemm_variant(variant, config, M, N, K, dtype, A, lda, B, ldb, C, ldc,
                                     stream)


def migemm_gemm_ex(op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha, beta, c_dtype, C, ldc,
                   stream=None) -> int:
    return lib().migemm_gemm_ex(op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha, beta,
                                c_dtype, C, ldc, stream)


def migemm_gemm_ex_variant(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha,
                           beta, c_dtype, C, ldc, stream=None) -> int:
    return lib().migemm_gemm_ex_variant(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B,
                                        ldb, alpha, beta, c_dtype, C, ldc, stream)


def migemm_gemm_ws(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha, beta,
                   c_dtype, C, ldc, workspace, workspace_bytes, stream=None) -> int:
    return lib().migemm_gemm_ws(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb,
                                alpha, beta, c_dtype, C, ldc, workspace, workspace_bytes, stream)


def migemm_gemm_noalloc(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha,
                        beta, c_dtype, C, ldc, stream=None) -> int:
    return lib().migemm_gemm_noalloc(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb,
                                     alpha, beta, c_dtype, C, ldc, stream)


def migemm_workspace_size(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb):
    """(status, bytes) of the workspace migemm_gemm_ws would use."""
    n = ctypes.c_int64(-1)
    st = lib().migemm_workspace_size(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb,
                                     ctypes.byref(n))
    return st, n.value


def _parse_description(text: str) -> dict:
    out = {}
    for item in text.split(";"):
        if "=" in item:
            k, v = item.split("=", 1)
            out[k] = int(v) if v.lstrip("-").isdigit() else v
    return out


def migemm_describe(M, N, K, dtype, lda, ldb, ldc, buflen=8192):
    """(status, text) describing what migemm_gemm would run."""
    buf = ctypes.create_string_buffer(buflen)
    st = lib().migemm_describe(M, N, K, dtype, lda, ldb, ldc, buf, buflen)
    return st, buf.value.decode()


def migemm_describe_ex(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, c_dtype,
                       ldc, workspace_bytes, buflen=8192):
    """(status, text) describing what migemm_gemm_ws would run."""
    buf = ctypes.create_string_buffer(buflen)
    st = lib().migemm_describe_ex(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb,
                                  c_dtype, ldc, workspace_bytes, buf, buflen)
    return st, buf.value.decode()


def describe(*args, **kw) -> dict:
    """migemm_describe_ex's text parsed into a dict (integers where numeric)."""
    st, text = migemm_describe_ex(*args, **kw)
    if st != OK:
        raise MigemmError(st, "migemm_describe_ex")
    return _parse_description(text)


def migemm_convert(src_dtype, dst_dtype, rows, cols, src, lds, dst, ldd, stream=None) -> int:
    return lib().migemm_convert(src_dtype, dst_dtype, rows, cols, src, lds, dst, ldd, stream)


def migemm_variant_count() -> int:
    return lib().migemm_variant_count()


def migemm_variant_name(variant: int) -> str | None:
    s = lib().migemm_variant_name(variant)
    return s.decode() if s is not None else None


def migemm_variant_supports(variant: int, dtype: int) -> bool:
    return bool(lib().migemm_variant_supports(variant, dtype))


def migemm_config_count(variant: int) -> int:
    return lib().migemm_config_count(variant)


def migemm_config_name(variant: int, config: int) -> str | None:
    s = lib().migemm_config_name(variant, config)
    return s.decode() if s is not None else None


def migemm_select(M, N, K, dtype, A, lda, B, ldb, C, ldc):
    """(status, variant, config) that migemm_gemm would use."""
    v, c = ctypes.c_int(-9), ctypes.c_int(-9)
    st = lib().migemm_select(M, N, K, dtype, A, lda, B, ldb, C, ldc, ctypes.byref(v),
                             ctypes.byref(c))
    return st, v.value, c.value


def migemm_status_string(status: int) -> str:
    return lib().migemm_status_string(status).decode()


def migemm_last_hip_error() -> int:
    return lib().migemm_last_hip_error()


def migemm_version() -> int:
    return lib().migemm_version()


# ---------------------------------------------------------- torch convenience

def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8,
             torch.int32: I32}
    if t.dtype not in codes:
        raise ValueError(f"unsupported dtype {t.dtype}; expected float32, float16, bfloat16, "
                         "int8 (operands) or int32 (output of an int8 product)")
    return codes[t.dtype]


def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("operands must be 2-D")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("operands must have unit stride along rows (row-major)")
    return max(1, t.stride(0) if t.shape[0] > 1 else t.shape[1])


def _operand(t):
    """(op, ld) of a 2-D operand: row-major (unit column stride) is OP_N with
    ld = stride(0); a transposed view (unit row stride) is OP_T with ld = stride(1)."""
    if t.dim() != 2:
        raise ValueError("operands must be 2-D")
    rows, cols = t.shape
    if cols <= 1 or t.stride(1) == 1:
        return OP_N, max(1, t.stride(0) if rows > 1 else cols)
    if rows <= 1 or t.stride(0) == 1:
        return OP_T, max(1, t.stride(1) if cols > 1 else rows)
    raise ValueError("operands must be row-major or transposed views of row-major storage")


def convert(src, dtype, out=None, *, stream=None):
    """``src`` (a 2-D CUDA tensor, float32/float16/bfloat16, unit column stride)
    converted to ``dtype`` on the GPU (round to nearest even when narrowing);
    ``out`` is allocated if not given.  Returns ``out`` without synchronising."""
    import torch
    if src.device.type != "cuda":
        raise ValueError("src must be on the GPU")
    rows, cols = src.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=src.device)
    elif out.dtype != dtype or tuple(out.shape) != (rows, cols):
        raise ValueError("out must have src's shape and the requested dtype")
    if stream is None:
        stream = torch.cuda.current_stream(src.device).cuda_stream
    st = migemm_convert(_dtype_code(src), _dtype_code(out), rows, cols, src.data_ptr() or None,
                        _ld(src), out.data_ptr() or None, _ld(out), stream)
    if st != OK:
        raise MigemmError(st, "migemm_convert")
    return out


def _check_device(name, t, device):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the operands on {device}")


def workspace(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, device):
    """A torch byte tensor on `device` large enough for migemm_gemm_ws with these
    arguments (None when the call needs none)."""
    import torch
    st, n = migemm_workspace_size(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb)
    if st != OK:
        raise MigemmError(st, "migemm_workspace_size")
    if n == 0:
        return None
    # torch's allocations are 512-byte aligned, beyond the 256 the library asks
    return torch.empty(n, dtype=torch.uint8, device=device)


def gemm(a, b, out=None, *, alpha: float = 1.0, beta: float = 0.0, out_dtype=None,
         variant: int = VARIANT_AUTO, config: int = -1, stream=None):
    """out = alpha * (A x B) + beta * out on the GPU for torch tensors.

    ``a`` (M x K) and ``b`` (K x N) are CUDA tensors of the same dtype
    (float32, float16, bfloat16, or int8 with an int32 ``out``) on one device,
    each row-major or a transposed view of row-major storage (``x.t()``, or a
    column-major tensor), passed as stored: no copy is made.  ``out`` (M x N,
    row-major, on the same device) may be float32, float16 or bfloat16; if not
    given it is allocated with ``out_dtype`` (default float32), which beta == 0
    requires.  The workspace the call asks for (migemm_workspace_size) is
    allocated by torch on the same stream and lent to migemm_gemm_ws.  Runs on
    ``stream`` (default: torch's current stream) and returns ``out`` without
    synchronising.
    """
    import torch
    device = a.device
    _check_device("a", a, device)
    _check_device("b", b, device)
    if a.dtype != b.dtype:
        raise ValueError(f"dtype mismatch: {a.dtype} vs {b.dtype}")
    dt = _dtype_code(a)
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} x {tuple(b.shape)}")
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing out")
        default = torch.int32 if a.dtype == torch.int8 else torch.float32
        out = torch.empty((M, N), dtype=out_dtype or default, device=device)
    else:
        _check_device("out", out, device)
        if tuple(out.shape) != (M, N) or (out_dtype is not None and out.dtype != out_dtype):
            raise ValueError("out must have shape (M, N) (and out_dtype, if given)")
    cd = _dtype_code(out)
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    pa, pb, pc = a.data_ptr() or None, b.data_ptr() or None, out.data_ptr() or None
    (op_a, lda), (op_b, ldb) = _operand(a), _operand(b)
    ws = workspace(variant, config, op_a, op_b, M, N, K, dt, pa, lda, pb, ldb, device)
    if ws is not None and stream != torch.cuda.current_stream(device).cuda_stream:
        # the block goes back to torch's pool when `ws` dies; keep it from being
        # reused before the work queued on `stream` has finished
        ws.record_stream(torch.cuda.ExternalStream(stream, device=device))
    st = migemm_gemm_ws(variant, config, op_a, op_b, M, N, K, dt, pa, lda, pb, ldb,
                        float(alpha), float(beta), cd, pc, _ld(out),
                        ws.data_ptr() if ws is not None else None,
                        ws.numel() if ws is not None else 0, stream)
    if st != OK:
        raise MigemmError(st, "migemm_gemm_ws")
    return out
