"""Seeded random cases against the oracle: shapes, storage and output forms drawn
together, so that combinations the targeted tests do not list are met too.

Each case draws the element type (FP32, FP16, BF16), M, N and K (biased towards
multiples of 8, 64 and 128 and one either side of them, where the kernels change
path: whole chunks, whole k-tiles, the partial last k-tile), the layout of A and
of B, padded leading dimensions and element offsets (offsets of 1 or 3 put an
operand off its 16-byte boundary), and the output form (plain FP32, or
alpha * A x B + beta * C into FP32, FP16 or BF16 with a padded, offset C).  The
call runs either through the automatic selection, with or without a workspace,
or on one configuration of the variant picked at random.  Every element is
compared with the oracle at the usual tolerance, and the padding around C must
stay untouched (it is NaN-filled).
"""
import numpy as np
import pytest
import torch

import dense_gemm_16_amd as mg
from dense_gemm_16_amd import inputs
from gpu_helpers import check_ex, oracle_ref, padding_untouched, run_gemm_ex, say

pytestmark = pytest.mark.gpu

CODES = {"f32": 0, "f16": 1, "bf16": 2}
TORCH_C = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}


def _dim(rng, hi):
    """A size in [1, hi]: a multiple of 8 (40%), one next to or on a multiple of 8,
    64 or 128 (30%), or any size."""
    u = rng.random()
    if u < 0.4:
        return 8 * int(rng.integers(1, hi // 8 + 1))
    if u < 0.7:
        m = int(rng.choice([8, 64, 128]))
        base = m * int(rng.integers(1, max(2, hi // m)))
        return int(min(hi, max(1, base + int(rng.integers(-1, 2)))))
    return int(rng.integers(1, hi + 1))


def _case(rng):
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    M, N, K = _dim(rng, 700), _dim(rng, 700), _dim(rng, 1200)
    ta, tb = bool(rng.random() < 0.3), bool(rng.random() < 0.3)
    pad = lambda: int(rng.choice([0, 0, 0, 0, 8, 8, 1, 3, 9]))
    lda = (M if ta else K) + pad()
    ldb = (K if tb else N) + pad()
    a_off = int(rng.choice([0, 0, 0, 0, 0, 0, 1, 3]))
    b_off = int(rng.choice([0, 0, 0, 0, 0, 0, 1, 3]))
    general = bool(rng.random() < 0.4)
    if general:
        alpha = float(rng.choice([1.0, 0.5, -1.25]))
        beta = float(rng.choice([0.0, 1.0, -0.75]))
        c_code = int(rng.choice([0, 1, 2]))
    else:
        alpha, beta, c_code = 1.0, 0.0, 0
    ldc = N + pad()
    c_off = int(rng.choice([0, 0, 1]))
    route = str(rng.choice(["auto", "auto_ws", "config"]))
    variant, config = -1, -1
    if route == "config":
        code = CODES[dtype]
        variants = [v for v in range(mg.migemm_variant_count()) if mg.migemm_variant_supports(v, code)
                    and v != mg.NAIVE]
        variant = int(rng.choice(variants))
        config = int(rng.integers(0, mg.migemm_config_count(variant)))
    return dict(dtype=dtype, M=M, N=N, K=K, ta=ta, tb=tb, lda=lda, ldb=ldb, a_off=a_off,
                b_off=b_off, alpha=alpha, beta=beta, c_code=c_code, ldc=ldc, c_off=c_off,
                route=route, variant=variant, config=config)


@pytest.mark.parametrize("block", range(8))
def test_random_cases_against_oracle(block):
    rng = np.random.default_rng(20261203 + block)
    for i in range(40):
        c = _case(rng)
        A, B = inputs.pair(c["M"], c["N"], c["K"], c["dtype"], "normal", seed=1000 * block + i)
        old = None
        if c["beta"] != 0.0:
            old = (torch.rand((c["M"], c["N"]), generator=torch.Generator().manual_seed(i))
                   - 0.5).to(TORCH_C[c["c_code"]])
        say(f"random block {block} case {i}: {c}")
        C, buf, mask = run_gemm_ex(A, B, c["dtype"], c["alpha"], c["beta"], c["c_code"], old,
                                   variant=c["variant"], config=c["config"], ldc=c["ldc"],
                                   c_off=c["c_off"], ta=c["ta"], tb=c["tb"], lda=c["lda"],
                                   ldb=c["ldb"], a_off=c["a_off"], b_off=c["b_off"],
                                   ws=None if c["route"] == "auto" else "auto")
        check_ex(C, A, B, c["dtype"], c["alpha"], c["beta"], c["c_code"], old,
                 ref=oracle_ref(A, B, c["dtype"]))
        assert padding_untouched(buf, mask), c
