"""Matrix-core throughput with no memory traffic, by operand values.

Runs the probe library's mfma_ceiling kernel (8 independent accumulator chains
per wave, two waves per SIMD, 1024 workgroups) for v_mfma_f32_32x32x16_bf16 and
v_mfma_f32_16x16x32_bf16 on zero operands and on random operand bits, and prints
TFLOP/s.  The gap between the two is the chip's power management: the
instruction takes the same cycles, but switching random bits draws enough power
to lower the clock.

    python3 tests/probes/mfma_ceiling.py
"""
import ctypes
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    L = ctypes.CDLL(os.path.join(HERE, "libprobes.so"))
    L.probe_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p]
    blocks, iters = 1024, 4096
    out = torch.empty(blocks * 512, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for mf in (32, 16):
        k = 16 if mf == 32 else 32
        n = iters if mf == 32 else 2 * iters
        flop = blocks * 8 * n * 8 * 2 * mf * mf * k
        for mode, label in ((0, "zero operands"), (2, "random operands")):
            def f():
                if L.probe_mfma_ceiling(mf, out.data_ptr(), blocks, n, mode, s) != 0:
                    raise RuntimeError("probe launch failed")
            for _ in range(3):
                f()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(10):
                f()
            t1.record()
            t1.synchronize()
            ms = t0.elapsed_time(t1) / 10
            print(f"v_mfma_f32_{mf}x{mf}x{k}_bf16 {label:16s}: {ms:.3f} ms  "
                  f"{flop / ms / 1e9:.1f} TFLOP/s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
