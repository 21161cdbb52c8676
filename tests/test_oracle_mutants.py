"""Planted mistakes in the oracle must fail its pins (CPU only).

Each mutant is a copy of ``oracle/oracle.c`` with one plausible mistake (a
dropped term, a wrong exponent bias, a shifted index, a lost absolute value,
a wrong sign), built into a temporary library.  The pins of
``test_oracle.py`` are re-run as predicates against the mutant; every mutant
must fail at least one of them, and the unmodified source must pass all.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from dense_gemm_16_amd import inputs

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "none": [],
    "drop_last_k": [("for (int64_t k = 0; k < K; ++k) {\n            const double a",
                     "for (int64_t k = 0; k < K - 1; ++k) {\n            const double a"),
                    ("for (int64_t k = 0; k < K; ++k) {\n            const double p",
                     "for (int64_t k = 0; k < K - 1; ++k) {\n            const double p")],
    "f16_bias": [("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)")],
    "f16_subnormal": [("ldexp((double)f, -24)", "ldexp((double)f, -25)")],
    "bf16_fraction": [("ldexp((double)(128 + f), e - 134)", "ldexp((double)(256 + f), e - 135)")],
    "shifted_column": [("c[j] += p;", "c[(j + 1) % N] += p;"),
                       ("const double p = decode_at(A, dtype, i * lda + k) * decode_at(B, dtype, k * ldb + j);",
                        "const double p = decode_at(A, dtype, i * lda + k) * decode_at(B, dtype, k * ldb + (j + 1) % N);")],
    "transposed_b": [("Bd[k * N + j] = decode_at(B, dtype, k * ldb + j);",
                      "Bd[k * N + j] = decode_at(B, dtype, (j % K) * ldb + (k % N));"),
                     ("decode_at(B, dtype, k * ldb + j);\n            c += p;",
                      "decode_at(B, dtype, (j % K) * ldb + (k % N));\n            c += p;")],
    "scale_without_abs": [("s[j] += fabs(p);", "s[j] += p;"), ("s += fabs(p);", "s += p;")],
    "sign": [("c[j] += p;", "c[j] -= p;"), ("            c += p;", "            c -= p;")],
    "encode_ties_away": [("const double r = rint(ax / q) * q;", "const double r = round(ax / q) * q;")],
    "encode_truncate": [("const double r = rint(ax / q) * q;", "const double r = trunc(ax / q) * q;")],
    "encode_f16_bias": [("((e + 15) << 10)", "((e + 14) << 10)")],
    "encode_overflow_at_max": [("if (ax >= thresh)", "if (ax > maxv)")],
    "encode_f16_subnormal": [("a / ldexp(1.0, -24)", "a / ldexp(1.0, -25)")],
    "epilogue_drops_beta": [("out[e] = alpha * acc[e] + old;", "out[e] = alpha * acc[e];")],
    "epilogue_alpha_on_old": [("beta * decode_at(Cold, c_dtype, e)", "alpha * decode_at(Cold, c_dtype, e)")],
    "epilogue_scale_without_abs": [("fabs(alpha) * S[e] + fabs(old)", "fabs(alpha) * S[e] + old")],
    "i8_unsigned": [("return (double)((int)(b & 0x7f) - (int)(b & 0x80));", "return (double)b;")],
}


def _build(name, edits, tmp_path):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, f"mutant {name}: pattern not found: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", str(c),
                    "-lm", "-o", str(so)], check=True)
    return oracle.Oracle(str(so))


def _b(t):
    return inputs.to_bits(t)


def pin_decoders(o):
    allbits = np.arange(65536, dtype=np.uint16)
    for code, tdt in ((oracle.F16, torch.float16), (oracle.BF16, torch.bfloat16)):
        got = o.decode(allbits, code)
        want = torch.from_numpy(allbits.view(np.int16).copy()).view(tdt).double().numpy()
        fin = np.isfinite(want)
        if not np.array_equal(got[fin], want[fin]):
            return False
    return True


def pin_ones(o):
    for dt in ("f32", "f16", "bf16"):
        A = torch.ones(5, 7).to(inputs.TORCH_DTYPES[dt])
        B = torch.ones(7, 3).to(inputs.TORCH_DTYPES[dt])
        C, S = o.gemm(_b(A), _b(B), inputs.DTYPE_CODES[dt])
        if not (np.all(C == 7) and np.all(S == 7)):
            return False
    return True


def pin_permutation(o):
    n, p = 13, 9
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3))
    P = torch.zeros(n, n)
    P[torch.arange(n), perm] = 1.0
    for dt in ("f32", "f16", "bf16"):
        B = inputs.draw((n, p), dt, "normal", torch.Generator().manual_seed(4))
        C, _ = o.gemm(_b(P.to(inputs.TORCH_DTYPES[dt])), _b(B), inputs.DTYPE_CODES[dt])
        if not np.array_equal(C, B.double().numpy()[perm.numpy()]):
            return False
    return True


def pin_small_int(o):
    for dt in ("f32", "f16", "bf16"):
        A, B = inputs.pair(11, 14, 17, dt, "int", seed=5)
        a = A.double().numpy().astype(np.int64)
        b = B.double().numpy().astype(np.int64)
        C, S = o.gemm(_b(A), _b(B), inputs.DTYPE_CODES[dt])
        if not (np.array_equal(C, (a @ b).astype(float))
                and np.array_equal(S, (np.abs(a) @ np.abs(b)).astype(float))):
            return False
    return True


def pin_subnormal_inputs(o):
    # binary16 subnormals times 1: C must equal the subnormal values exactly
    sub = torch.from_numpy(np.arange(1, 9, dtype=np.int16)).view(torch.float16).view(8, 1)
    one = torch.ones(1, 1, dtype=torch.float16)
    C, _ = o.gemm(_b(sub), _b(one), oracle.F16)
    return np.array_equal(C[:, 0], sub.double().numpy()[:, 0])


def pin_encode_roundtrip_and_ties(o):
    allbits = np.arange(65536, dtype=np.uint16)
    for code in (oracle.F16, oracle.BF16):
        vals = o.decode(allbits, code)
        pats = allbits[np.isfinite(vals)]
        if not np.array_equal(o.encode(o.decode(pats, code), code), pats):
            return False
        pos = np.sort(pats[(pats & 0x8000) == 0])
        lo, hi = pos[:-1], pos[1:]
        mid = (o.decode(lo, code) + o.decode(hi, code)) / 2
        if not np.array_equal(o.encode(mid, code), np.where((lo & 1) == 0, lo, hi)):
            return False
    return True


def pin_encode_overflow(o):
    mx = (2 - 2 ** -7) * 2.0 ** 127
    return (o.encode([65519.99, 65520.0], oracle.F16).tolist() == [0x7BFF, 0x7C00]
            and o.encode([mx, mx + 2.0 ** 119 * 0.999], oracle.BF16).tolist() == [0x7F7F, 0x7F7F])


def pin_epilogue_integers(o):
    g = np.random.default_rng(5)
    a = g.integers(-4, 5, (6, 9))
    b = g.integers(-4, 5, (9, 7))
    old = g.integers(-20, 21, (6, 7))
    A, B = torch.from_numpy(a).half(), torch.from_numpy(b).half()
    acc, S = o.gemm(_b(A), _b(B), oracle.F16)
    out, sc = o.epilogue(acc, S, 3.0, -2.0, oracle.F16, _b(torch.from_numpy(old).half()))
    return (np.array_equal(out, (3 * (a @ b) - 2 * old).astype(float))
            and np.array_equal(sc, (3 * (np.abs(a) @ np.abs(b)) + 2 * np.abs(old)).astype(float)))


def pin_i8(o):
    allb = np.arange(256, dtype=np.uint8)
    if not np.array_equal(o.decode(allb, oracle.I8), allb.view(np.int8).astype(np.float64)):
        return False
    g = np.random.default_rng(2)
    A = g.integers(-128, 128, (9, 40)).astype(np.int8)
    B = g.integers(-128, 128, (40, 11)).astype(np.int8)
    C, _ = o.gemm(A, B, oracle.I8)
    return np.array_equal(C, (A.astype(np.int64) @ B.astype(np.int64)).astype(float))


PINS = [pin_decoders, pin_ones, pin_permutation, pin_small_int, pin_subnormal_inputs, pin_i8,
        pin_encode_roundtrip_and_ties, pin_encode_overflow, pin_epilogue_integers]


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_fails_some_pin(name, tmp_path):
    o = _build(name, MUTANTS[name], tmp_path)
    results = {p.__name__: p(o) for p in PINS}
    if name == "none":
        assert all(results.values()), results
    else:
        assert not all(results.values()), f"mutant {name} passed every pin: {results}"
