// regtile_valu.hip -- FP32 GEMM with register micro-tiles on VALU FMA.
//
// The design of page "matmul_registers.cu" (matmulRegTile2d and
// matmulRegTile2dVec4): a BM x BN workgroup tile, each work-item owning a
// TM x TN micro-tile of accumulators in registers, per k step TM values of A
// and TN values of B read from LDS and reused TN and TM times; 16-byte global
// loads; the A tile stored k-major (transposed) in LDS so a work-item's TM
// values of A are contiguous; 16-byte LDS reads and 16-byte C stores.
//
// gfx950 changes:
// * Double-buffered LDS with register prefetch: the next k-tile's global
//   loads are issued before the current k-tile's FMAs and written to the
//   other LDS buffer after them, so one barrier per k-tile remains.
// * Conflict-free 16-byte LDS reads for wave64: a work-item's micro-tile
//   columns are TN/4 groups of 4, strided by BN/TN groups (and likewise for
//   rows), so the 16 work-items of a wavefront that differ in column read 16
//   consecutive 16-byte words.
// * Scalar v_fma_f32 only (packed FP32 instructions are disabled for this
//   build), so the VALU ceiling is 128 FLOP/clock/CU: 78.6 TFLOP/s at
//   2.4 GHz, half the FP32 matrix-core rate.
// * Every edge is guarded: tiles inside the matrix take unguarded vector
//   loads; edge tiles and the K tail load zeros out of range; rows not 16-byte
//   aligned are read element by element.
// * Either operand may be given transposed.  Both LDS tiles are k-major, so an
//   operand stored with its M or N side contiguous (row-major B, or A given
//   transposed) is copied row for row, and one stored with k contiguous
//   (row-major A, or B given transposed) is transposed on its way into LDS.
#include "common.hpp"

namespace migemm {
namespace {

__device__ __forceinline__ f32x4 ld4_guarded(const float* __restrict__ base, int64_t r,
                                             int64_t c0, int64_t nrows, int64_t ncols,
                                             int64_t ld, bool vec_ok) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r >= nrows) return v;
    const float* p = base + r * ld + c0;
    if (vec_ok && c0 + 4 <= ncols) return *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (c0 + e < ncols) ? p[e] : 0.f;
    return v;
}

// One operand's BX x BK tile into a k-major LDS tile img[BK][LD].  KC: stored
// with k contiguous (transposed on the way in); otherwise stored with the BX
// side contiguous (copied as 16-byte row pieces).
template <int BX, int BK, int NT, int LD, bool KC>
struct ValuStage {
    static constexpr int UNITS = BX * BK / 4;
    static constexpr int PER = (UNITS + NT - 1) / NT;
    f32x4 r[PER];

    // Tile rows x0.. (of ext) and k0.. (of K); p and ld as stored.
    __device__ __forceinline__ void load(const float* __restrict__ p, int64_t ld, int tid,
                                         int64_t x0, int64_t k0, int64_t ext, int64_t K,
                                         bool fast, bool vec) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int id = tid + q * NT;
            if (UNITS % NT != 0 && id >= UNITS) continue;
            if constexpr (KC) {
                const int64_t x = x0 + id / (BK / 4), k = k0 + (id % (BK / 4)) * 4;
                r[q] = (fast && vec) ? *reinterpret_cast<const f32x4*>(p + x * ld + k)
                                     : ld4_guarded(p, x, k, ext, K, ld, vec);
            } else {
                const int64_t k = k0 + id / (BX / 4), x = x0 + (id % (BX / 4)) * 4;
                r[q] = (fast && vec) ? *reinterpret_cast<const f32x4*>(p + k * ld + x)
                                     : ld4_guarded(p, k, x, K, ext, ld, vec);
            }
        }
    }

    __device__ __forceinline__ void store(float (*img)[LD], int tid) const {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int id = tid + q * NT;
            if (UNITS % NT != 0 && id >= UNITS) continue;
            if constexpr (KC) {
                const int x = id / (BK / 4), kc = id % (BK / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) img[kc * 4 + e][x] = r[q][e];
            } else {
                const int kr = id / (BX / 4), xc = id % (BX / 4);
                *reinterpret_cast<f32x4*>(&img[kr][xc * 4]) = r[q];
            }
        }
    }
};

template <int BM, int BN, int BK, int TM, int TN, bool GEN, bool TA, bool TB>
__global__ __launch_bounds__((BM / TM) * (BN / TN)) void regtile_valu_kernel(
    int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
    const float* __restrict__ B, int64_t ldb, Epi out, bool av, bool bv, bool cv,
    unsigned tiles_n) {
    constexpr int NC = BN / TN, NR = BM / TM, NT = NC * NR;
    constexpr int PAD = 4;  // keeps k-major A rows 16-byte aligned while shifting banks
    static_assert(TM % 4 == 0 && TN % 4 == 0 && BK % 4 == 0, "16-byte groups");

    __shared__ __attribute__((aligned(16))) float sAt[2][BK][BM + PAD];
    __shared__ __attribute__((aligned(16))) float sB[2][BK][BN + PAD];

    const int tid = threadIdx.x;
    const int tc = tid % NC, tr = tid / NC;
    const int64_t m0 = static_cast<int64_t>(blockIdx.x / tiles_n) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x % tiles_n) * BN;
    const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

    // A is k-contiguous unless given transposed; B only when given transposed.
    ValuStage<BM, BK, NT, BM + PAD, !TA> stA;
    ValuStage<BN, BK, NT, BN + PAD, TB> stB;
    auto load_tile = [&](int64_t k0) {
        const bool fast = full_mn && (k0 + BK <= K);
        stA.load(A, lda, tid, m0, k0, M, K, fast, av);
        stB.load(B, ldb, tid, n0, k0, N, K, fast, bv);
    };
    auto store_tile = [&](int buf) {
        stA.store(sAt[buf], tid);
        stB.store(sB[buf], tid);
    };

    const int64_t KT = ceil_div(K, BK);
    if (KT > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        if (kt + 1 < KT) load_tile((kt + 1) * BK);
#pragma unroll
        for (int p = 0; p < BK; ++p) {
            float a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM / 4; ++i) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(&sAt[cur][p][4 * (tr + i * NR)]);
                a[4 * i] = v[0]; a[4 * i + 1] = v[1]; a[4 * i + 2] = v[2]; a[4 * i + 3] = v[3];
            }
#pragma unroll
            for (int j = 0; j < TN / 4; ++j) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(&sB[cur][p][4 * (tc + j * NC)]);
                b[4 * j] = v[0]; b[4 * j + 1] = v[1]; b[4 * j + 2] = v[2]; b[4 * j + 3] = v[3];
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < KT) store_tile(cur ^ 1);
        __syncthreads();
    }

    // Row 4*(tr + i*NR) + ii, columns 4*(tc + j*NC) .. +3.
#pragma unroll
    for (int i = 0; i < TM / 4; ++i) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int64_t row = m0 + 4 * (tr + i * NR) + ii;
            if (!full_mn && row >= M) continue;
#pragma unroll
            for (int j = 0; j < TN / 4; ++j) {
                const int64_t col = n0 + 4 * (tc + j * NC);
                f32x4 v = {acc[4 * i + ii][4 * j], acc[4 * i + ii][4 * j + 1],
                           acc[4 * i + ii][4 * j + 2], acc[4 * i + ii][4 * j + 3]};
                const int64_t idx = row * out.ldc + col;
                if (!GEN && cv && (full_mn || col + 4 <= N)) {
                    *reinterpret_cast<f32x4*>(static_cast<float*>(out.C) + idx) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < N) store_out<GEN>(out, idx + e, v[e]);
                }
            }
        }
    }
}

template <int BM, int BN, int BK, int TM, int TN, bool GEN, bool TA, bool TB>
hipError_t launch_gen(const GemmArgs& g) {
    const int64_t gx = ceil_div(g.N, BN), gy = ceil_div(g.M, BM);
    if (gx * gy > 0x7fffffff) return hipErrorInvalidValue;
    const bool av = aligned16(g.A) && g.lda % 4 == 0;
    const bool bv = aligned16(g.B) && g.ldb % 4 == 0;
    const bool cv = aligned16(g.out.C) && g.out.ldc % 4 == 0;
    return launch_kernel(g, regtile_valu_kernel<BM, BN, BK, TM, TN, GEN, TA, TB>,
                         dim3(static_cast<unsigned>(gx * gy)), dim3((BM / TM) * (BN / TN)), g.M,
                         g.N, g.K, static_cast<const float*>(g.A), g.lda,
                         static_cast<const float*>(g.B), g.ldb, g.out, av, bv, cv,
                         static_cast<unsigned>(gx));
}

template <int BM, int BN, int BK, int TM, int TN, bool GEN>
hipError_t launch_layout(const GemmArgs& g) {
    if (g.ta)
        return g.tb ? launch_gen<BM, BN, BK, TM, TN, GEN, true, true>(g)
                    : launch_gen<BM, BN, BK, TM, TN, GEN, true, false>(g);
    return g.tb ? launch_gen<BM, BN, BK, TM, TN, GEN, false, true>(g)
                : launch_gen<BM, BN, BK, TM, TN, GEN, false, false>(g);
}

template <int BM, int BN, int BK, int TM, int TN>
hipError_t launch_cfg(const GemmArgs& g) {
    return g.general() ? launch_layout<BM, BN, BK, TM, TN, true>(g)
                       : launch_layout<BM, BN, BK, TM, TN, false>(g);
}

const char* const kNames[] = {"128x128x8 8x8", "128x128x16 8x8", "64x64x16 4x4",
                              "128x64x16 8x4"};

}  // namespace

int regtile_valu_config_count() { return 4; }
const char* regtile_valu_config_name(int c) { return (c >= 0 && c < 4) ? kNames[c] : nullptr; }

hipError_t launch_regtile_valu(const GemmArgs& g, int config) {
    switch (config) {
        case 1: return launch_cfg<128, 128, 16, 8, 8>(g);
        case 2: return launch_cfg<64, 64, 16, 4, 4>(g);
        case 3: return launch_cfg<128, 64, 16, 8, 4>(g);
        default: return launch_cfg<128, 128, 8, 8, 8>(g);
    }
}

}  // namespace migemm
