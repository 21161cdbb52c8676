"""Comparison of a GPU result against the oracle -- TEST INFRASTRUCTURE ONLY.

Rule, per element (i, j), with C_ref and S = sum_k |A[i][k] * B[k][j]| from the
oracle in binary64:

* exact mode (inputs whose every partial sum is an integer below 2^24, and the
  structured identity / permutation / all-ones cases): the GPU value must equal
  C_ref as a number (+0 == -0);
* otherwise |C - C_ref| <= tol * S, with tol = 1e-4 when the inputs are FP32 and
  5e-4 when they are FP16 or BF16 with FP32 accumulation; where S == 0 the two
  must be equal.

S is the scale of the standard forward error bound of a dot product: a sum of
K products accumulated in binary32 (each product of two FP16/BF16 values is
exact in binary32) is off by at most about K * 2^-24 * S, so cancellation in
C_ref never makes the rule unfair.  The first failing element is reported with
its row and column, in the manner of the first-mismatch report on page
"matmul_registers.cu".

A result stored in a narrower format (``out_dtype`` FP16 or BF16, or FP32 after
the scaled update) is also off by its final rounding: at most half a unit in the
last place, u |C| with u = 2^-24, 2^-11, 2^-8 for FP32, FP16, BF16, or half the
smallest subnormal (2^-150, 2^-25, 2^-134) near zero.  With ``out_dtype`` given
the bound is tol * S * (1 + u) + u |C_ref| + that half subnormal, where S is the
scale of the whole update (|alpha| S + |beta C_old| from the oracle).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TOL_F32 = 1e-4
TOL_HALF = 5e-4
# unit roundoff and half the smallest subnormal of each stored format
OUT_UNIT = {0: 2.0 ** -24, 1: 2.0 ** -11, 2: 2.0 ** -8}
OUT_TINY = {0: 2.0 ** -150, 1: 2.0 ** -25, 2: 2.0 ** -134}


def tolerance(dtype: int) -> float:
    return TOL_F32 if dtype == 0 else TOL_HALF


@dataclass
class CheckResult:
    ok: bool
    n_bad: int
    max_ratio: float          # max |C - C_ref| / S over elements with S > 0
    first: tuple | None       # (row, col, got, want, S) of the first failure

    def __str__(self) -> str:
        if self.ok:
            return f"ok (max |err|/S = {self.max_ratio:.3e})"
        r, c, got, want, s = self.first
        return (f"{self.n_bad} bad elements; first at row {r} col {c}: got {got!r} want {want!r}"
                f" S={s!r}; max |err|/S = {self.max_ratio:.3e}")


def compare(got, want, scale, tol: float | None = None, exact: bool = False,
            out_dtype: int | None = None) -> CheckResult:
    """Compare ``got`` (GPU, any float array) with ``want``/``scale`` (oracle, float64);
    ``out_dtype`` adds the final rounding of a result stored in that format."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    if got.shape != want.shape or want.shape != scale.shape:
        raise ValueError(f"shape mismatch: {got.shape} {want.shape} {scale.shape}")
    err = np.abs(got - want)
    finite = np.isfinite(got)
    if exact:
        bad = ~(finite & (got == want))
    else:
        if tol is None:
            raise ValueError("tol is required unless exact=True")
        if out_dtype is None:
            bound = tol * scale
        else:
            u = OUT_UNIT[out_dtype]
            bound = tol * scale * (1.0 + u) + u * np.abs(want) + OUT_TINY[out_dtype]
        bad = ~(finite & (err <= bound))
        bad |= (scale == 0) & (got != want)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), 0.0)
    ratio = np.where(finite, ratio, np.inf)
    max_ratio = float(ratio.max()) if ratio.size else 0.0
    n_bad = int(bad.sum())
    first = None
    if n_bad:
        flat = int(np.flatnonzero(bad.reshape(-1))[0])
        idx = np.unravel_index(flat, bad.shape) if bad.ndim > 1 else (flat,)
        row = int(idx[0])
        col = int(idx[1]) if len(idx) > 1 else -1
        first = (row, col, float(got[idx]), float(want[idx]), float(scale[idx]))
    return CheckResult(ok=(n_bad == 0), n_bad=n_bad, max_ratio=max_ratio, first=first)
