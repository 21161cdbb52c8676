// skinny16.hip -- FP16/BF16 products with at most 16 rows of C (M <= 16): the
// last few rows of a product whose row count is just past a whole number of
// tile bands (a 2050-row product: rows 2048 and 2049).
//
// The same C = A x B with FP32 sums (page "CUDA-Practice 09", section on FP32
// accumulation), shaped for a short, wide C: one workgroup per 16 columns of C,
// its waves (sixteen or eight, see Shape) splitting K between them.  Each wave
// takes every sixteenth (eighth) 32-deep k-step and runs one
// v_mfma_f32_16x16x32 per step, with the fragments
// loaded straight from global memory into registers (16 bytes per lane where the
// operand is k-contiguous, eight 2-byte loads where it is not); rows of A past M
// and k past K read as zeros, and columns of B past N are clamped (their outputs
// are not stored).  The waves' partial 16 x 16 blocks are then summed through
// LDS in wave order, so the result does not depend on timing.  A 128x128-tile
// launch would instead walk all of K for two rows of C on 32 workgroups.
//
// A k-contiguous operand needs K a multiple of 8 (or to be a copy zero-filled to
// one), so that each lane's 8-deep run of k can be read whole; the launcher
// returns hipErrorInvalidValue otherwise.
#include "mfma_gemm.hpp"

namespace migemm {
namespace {

// Both operands k-contiguous: sixteen waves of five k-steps per round (a lane
// holds 40 registers of fragments).  Otherwise eight waves of four k-steps: the
// strided 2-byte loads of an operand stored with k as its row index need more
// address registers than sixteen waves per workgroup leave each lane.
template <bool TA, bool TB> struct Shape {
    static constexpr bool KC = !TA && TB;
    static constexpr int kWaves = KC ? 16 : 8, kBatch = KC ? 5 : 4;
};

// The 16-byte k-run [k0, k0 + 8) of row `row` of a k-contiguous operand (kc:
// read whole, K being a multiple of 8 or the operand a copy zero-filled to one),
// or of column `row` of an operand stored with k as its row index (k-rows at or
// past K read as zeros).
template <typename E, bool KC>
__device__ __forceinline__ u32x4 krun(const E* __restrict__ p, int64_t ld, int64_t row,
                                      int64_t k0, int64_t K) {
    if constexpr (KC) {
        return *reinterpret_cast<const u32x4*>(p + row * ld + k0);
    } else {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(p) + k0 * ld + row;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = k0 + 2 * e < K ? q[(2 * e) * ld] : 0u;
            const uint32_t hi = k0 + 2 * e + 1 < K ? q[(2 * e + 1) * ld] : 0u;
            v[e] = lo | (hi << 16);
        }
        return v;
    }
}

// TA: A stored K x M; TB: B stored N x K (k contiguous).
template <typename E, bool GEN, bool TA, bool TB>
__global__ __launch_bounds__((Shape<TA, TB>::kWaves * kWave)) void skinny16_kernel(int64_t M, int64_t N, int64_t K,
                                                                  const E* __restrict__ A,
                                                                  int64_t lda,
                                                                  const E* __restrict__ B,
                                                                  int64_t ldb, Epi out) {
    using Op = MfmaOp<E, 16>;
    using L = AccLayout<16>;
    constexpr int kWaves = Shape<TA, TB>::kWaves, kBatch = Shape<TA, TB>::kBatch;
    __shared__ f32x4 part[kWaves][kWave];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int r = lane % 16, g = lane / 16;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t n = min(n0 + r, N - 1);  // B column fed by this lane (clamped)
    const bool a_in = r < M;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int64_t steps = ceil_div(K, 32);
    // kBatch of this wave's steps per round, all their loads issued before the
    // first matrix instruction: one memory latency per round instead of per step
    // (with both operands k-contiguous a K of up to 2560 takes one round)
    for (int64_t s0 = wave; s0 < steps; s0 += kBatch * kWaves) {
        u32x4 a[kBatch], b[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int64_t s = s0 + q * kWaves;
            a[q] = b[q] = u32x4{0u, 0u, 0u, 0u};
            const int64_t k0 = s * 32 + 8 * g;
            if (s < steps && k0 < K) {
                if (a_in) a[q] = krun<E, !TA>(A, lda, r, k0, K);
                b[q] = krun<E, TB>(B, ldb, n, k0, K);
            }
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) Op::run(acc, a[q], b[q]);
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    f32x4 sum = part[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        const f32x4 p = part[w][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[e] += p[e];
    }
    const int64_t col = n0 + L::col(lane);
    if (col >= N) return;
#pragma unroll
    for (int e = 0; e < L::R; ++e) {
        const int64_t row = L::row(lane, e);
        if (row < M) store_out<GEN>(out, row * out.ldc + col, sum[e]);
    }
}

template <typename E, bool GEN>
hipError_t launch_typed(const GemmArgs& g) {
    const dim3 grid(static_cast<unsigned>(ceil_div(g.N, 16)));
    const E* A = static_cast<const E*>(g.A);
    const E* B = static_cast<const E*>(g.B);
#define MIGEMM_LAUNCH(TA_, TB_)                                                                \
    return launch_kernel(g, skinny16_kernel<E, GEN, TA_, TB_>, grid,                          \
                         dim3(Shape<TA_, TB_>::kWaves * kWave), g.M, g.N, g.K, A, g.lda, B,   \
                         g.ldb, g.out)
    if (g.ta) {
        if (g.tb) MIGEMM_LAUNCH(true, true);
        MIGEMM_LAUNCH(true, false);
    }
    if (g.tb) MIGEMM_LAUNCH(false, true);
    MIGEMM_LAUNCH(false, false);
#undef MIGEMM_LAUNCH
}

}  // namespace

bool skinny16_fits(const GemmArgs& g) {
    // k-contiguous operands are read 16 bytes at a time: aligned rows in whole
    // chunks, K a multiple of 8 unless the operand is a zero-filled copy
    const bool k_whole = g.K % 8 == 0;
    const bool a_ok = g.ta || (aligned16(g.A) && g.lda % 8 == 0 && (k_whole || g.pad_a));
    const bool b_ok = !g.tb || (aligned16(g.B) && g.ldb % 8 == 0 && (k_whole || g.pad_b));
    return g.M >= 1 && g.M <= 16 && g.N >= 1 && g.K > 0 && a_ok && b_ok &&
           ceil_div(g.N, 16) <= 0x7fffffff && (g.dtype == 1 || g.dtype == 2);
}

hipError_t launch_skinny16(const GemmArgs& g) {
    if (!skinny16_fits(g)) return hipErrorInvalidValue;
    if (g.general())
        return g.dtype == 1 ? launch_typed<_Float16, true>(g) : launch_typed<bf16_t, true>(g);
    return g.dtype == 1 ? launch_typed<_Float16, false>(g) : launch_typed<bf16_t, false>(g);
}

}  // namespace migemm
