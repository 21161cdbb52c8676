"""CPU oracle for the dense matrix product -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and
shares no source with it.

The arithmetic lives in ``oracle.c`` (plain C, binary64): for A (M x K) and
B (K x N), row-major,

    C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]      (ascending k, binary64)
    S[i][j] = sum_{k=0}^{K-1} |A[i][k] * B[k][j]|

and, for the scaled update with a previous C (``epilogue``),

    out = alpha * C + beta * C_old,   scale = |alpha| S + |beta C_old|

with ``encode`` rounding binary64 values to FP32, FP16 or BF16 (nearest, ties
to even) for outputs stored in those formats.

following the element-wise definition on page "Tensor cores and matrix
operations" (section "Traditional Approach: Element-by-Element") and the fp64
CPU reference on page "matmul_registers.cu".  This module only marshals
numpy arrays into that library.

Inputs are passed as their stored encodings: ``float32`` arrays for FP32,
``uint16`` (or ``int16``) arrays of raw bits for FP16 and BF16, ``int8`` (or
``uint8``) arrays for INT8.  The oracle decodes the bits itself.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build, library_path

F32, F16, BF16, I8 = 0, 1, 2, 3
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16, "i8": I8}


class Oracle:
    """Handle on one build of the oracle library (the default build, or a test's mutant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_decode_array.argtypes = [i32, i64, vp, vp]
        lib.oracle_decode_array.restype = i32
        lib.oracle_max_threads.argtypes = [i32]
        lib.oracle_max_threads.restype = i32
        lib.oracle_gemm.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, vp, vp, i32]
        lib.oracle_gemm.restype = i32
        lib.oracle_gemm_entries.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, i64, vp, vp,
                                            vp, vp, i32]
        lib.oracle_gemm_entries.restype = i32
        lib.oracle_encode_array.argtypes = [i32, i64, vp, vp]
        lib.oracle_encode_array.restype = i32
        lib.oracle_epilogue.argtypes = [i64, ctypes.c_double, ctypes.c_double, i32, vp, vp, vp,
                                        vp, vp]
        lib.oracle_epilogue.restype = i32
        self.lib = lib
        self.path = path

    def threads_used(self, nthreads: int | None = None) -> int:
        """The thread count a call with ``nthreads`` actually runs with."""
        return int(self.lib.oracle_max_threads(int(nthreads or default_threads())))

    def decode(self, bits, dtype: int) -> np.ndarray:
        """Decode stored elements to exact float64 values (the oracle's own decoder)."""
        arr = np.ascontiguousarray(np.asarray(bits))
        if dtype == F32:
            arr = arr if arr.dtype == np.float32 else arr.view(np.float32)
        elif dtype == I8:
            arr = arr.view(np.uint8)
        elif arr.dtype == np.int16:
            arr = arr.view(np.uint16)
        out = np.empty(arr.shape, dtype=np.float64)
        st = self.lib.oracle_decode_array(dtype, arr.size, _ptr(arr), _ptr(out))
        if st:
            raise ValueError(f"oracle_decode_array failed with status {st}")
        return out

    def encode(self, values, dtype: int) -> np.ndarray:
        """Round float64 values to the stored format, nearest with ties to even (the
        oracle's own encoder): float32 for FP32, raw uint16 bits for FP16 and BF16."""
        v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
        out = np.empty(v.shape, dtype=np.uint32 if dtype == F32 else np.uint16)
        st = self.lib.oracle_encode_array(dtype, v.size, _ptr(v), _ptr(out))
        if st:
            raise ValueError(f"oracle_encode_array failed with status {st}")
        return out.view(np.float32) if dtype == F32 else out

    def epilogue(self, acc, S, alpha: float, beta: float, c_dtype: int, c_old=None):
        """out = alpha * acc + beta * C_old and scale = |alpha| S + |beta C_old|, element
        by element in float64.  c_old holds the previous C in its stored format (float32
        or raw uint16 bits) with acc's shape; it is not read when beta == 0."""
        acc = np.ascontiguousarray(np.asarray(acc, dtype=np.float64))
        S = np.ascontiguousarray(np.asarray(S, dtype=np.float64))
        if S.shape != acc.shape:
            raise ValueError("acc and S differ in shape")
        old = None
        if beta != 0.0:
            if c_old is None:
                raise ValueError("beta != 0 needs the previous C")
            old = np.asarray(c_old)
            if c_dtype == F32:
                old = old if old.dtype == np.float32 else old.view(np.float32)
            elif old.dtype == np.int16:
                old = old.view(np.uint16)
            old = np.ascontiguousarray(old)
            if old.shape != acc.shape:
                raise ValueError("previous C differs in shape from the product")
        out = np.empty_like(acc)
        scale = np.empty_like(acc)
        st = self.lib.oracle_epilogue(acc.size, float(alpha), float(beta), c_dtype,
                                      _ptr(old) if old is not None else None, _ptr(acc), _ptr(S),
                                      _ptr(out), _ptr(scale))
        if st:
            raise ValueError(f"oracle_epilogue failed with status {st}")
        return out, scale

    def gemm(self, A, B, dtype: int, nthreads: int | None = None, want_scale: bool = True):
        """Full product: (C, S) as float64 arrays of shape (M, N); S is None if not wanted."""
        A = _as_stored(A, dtype)
        B = _as_stored(B, dtype)
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError(f"inner dimensions differ: {A.shape} x {B.shape}")
        C = np.empty((M, N), dtype=np.float64)
        S = np.empty((M, N), dtype=np.float64) if want_scale else None
        st = self.lib.oracle_gemm(M, N, K, dtype, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(C),
                                  _ptr(S) if S is not None else None,
                                  int(nthreads or default_threads()))
        if st:
            raise ValueError(f"oracle_gemm failed with status {st}")
        return C, S

    def gemm_entries(self, A, B, dtype: int, rows, cols, nthreads: int | None = None):
        """C[rows[e], cols[e]] and S for selected entries, one dot product each."""
        A = _as_stored(A, dtype)
        B = _as_stored(B, dtype)
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError(f"inner dimensions differ: {A.shape} x {B.shape}")
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape or rows.ndim != 1:
            raise ValueError("rows and cols must be 1-D of equal length")
        n = rows.size
        C = np.empty(n, dtype=np.float64)
        S = np.empty(n, dtype=np.float64)
        st = self.lib.oracle_gemm_entries(M, N, K, dtype, _ptr(A), _ld(A), _ptr(B), _ld(B), n,
                                          _ptr(rows), _ptr(cols), _ptr(C), _ptr(S),
                                          int(nthreads or default_threads()))
        if st:
            raise ValueError(f"oracle_gemm_entries failed with status {st}")
        return C, S


_default: Oracle | None = None


def _oracle() -> Oracle:
    global _default
    if _default is None:
        path = library_path()
        if not os.path.exists(path):
            build()
        _default = Oracle(path)
    return _default


def default_threads() -> int:
    """Host threads to use: the CPUs this process may run on, capped by OMP_NUM_THREADS."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def threads_used(nthreads: int | None = None) -> int:
    return _oracle().threads_used(nthreads)


def decode(bits, dtype: int) -> np.ndarray:
    return _oracle().decode(bits, dtype)


def gemm(A, B, dtype: int, nthreads: int | None = None, want_scale: bool = True):
    return _oracle().gemm(A, B, dtype, nthreads, want_scale)


def encode(values, dtype: int) -> np.ndarray:
    return _oracle().encode(values, dtype)


def epilogue(acc, S, alpha: float, beta: float, c_dtype: int, c_old=None):
    return _oracle().epilogue(acc, S, alpha, beta, c_dtype, c_old)


def gemm_entries(A, B, dtype: int, rows, cols, nthreads: int | None = None):
    return _oracle().gemm_entries(A, B, dtype, rows, cols, nthreads)


def _as_stored(x, dtype: int) -> np.ndarray:
    x = np.asarray(x)
    if dtype == F32:
        if x.dtype != np.float32:
            raise TypeError(f"FP32 operand must be float32, got {x.dtype}")
    elif dtype == I8:
        if x.dtype not in (np.int8, np.uint8):
            raise TypeError(f"INT8 operand must be int8/uint8, got {x.dtype}")
        x = x.view(np.uint8)
    else:
        if x.dtype == np.int16:
            x = x.view(np.uint16)
        if x.dtype != np.uint16:
            raise TypeError(f"16-bit operand must be raw uint16/int16 bits, got {x.dtype}")
    if x.ndim != 2:
        raise ValueError("operands must be 2-D")
    if x.shape[1] > 1 and x.strides[1] != x.itemsize:
        x = np.ascontiguousarray(x)
    return x


def _ld(x: np.ndarray) -> int:
    if x.shape[0] <= 1:
        return max(1, x.shape[1])
    if x.strides[0] % x.itemsize:
        raise ValueError("row stride must be a whole number of elements")
    return max(1, x.strides[0] // x.itemsize)


def _ptr(x: np.ndarray):
    return x.ctypes.data if x.size else None


