// skinny.hip -- products with at most 16 rows of C (M <= 16), FP32, FP16/BF16
// or INT8 inputs: the last few rows (or, transposed, columns) of a product whose
// size is just past a whole number of tile bands (a 2050-row product: rows 2048
// and 2049).
//
// The same C = A x B with FP32 sums (page "CUDA-Practice 09", section on FP32
// accumulation; exact INT32 sums for INT8), shaped for a short, wide C: one
// workgroup per 16 columns of C, its waves (sixteen or eight, see Shape)
// splitting K between them.  A k-step is one 16-byte chunk per lane of each
// operand: 32 deep for 16-bit elements (one v_mfma_f32_16x16x32), 64 deep for
// INT8 (one v_mfma_i32_16x16x64_i8), 16 deep for FP32 (four
// v_mfma_f32_16x16x4_f32, element e of every lane's chunk feeding instruction
// e, the same k order for A and B).
// Each wave takes every sixteenth (eighth) k-step; rows of A past M and k past
// K read as zeros.  The waves' partial 16 x 16 blocks are then summed through
// LDS in wave order, so the result does not depend on timing.  A 128x128-tile
// launch would instead walk all of K for two rows of C on 32 workgroups.
//
// Every operand is read 16 bytes per lane, in one of two forms:
// * k-contiguous (row-major A, B given transposed): a lane's run of consecutive
//   k of its row or column is one 16-byte chunk, loaded straight into the
//   fragment;
// * k as the row index (row-major B, A given transposed): a step's k-rows x 16
//   columns are loaded as 64 chunks of 16 bytes, one per lane, written to a slot
//   of the wave's own LDS area as a row-major block, and read back transposed:
//   16-bit elements with two ds_read_b64_tr_b16, which hand each lane one column
//   of four k-rows apiece; INT8 with two ds_read_b64_tr_b8 (one column of eight
//   k-rows apiece); FP32 with four 4-byte reads, one per k-row (k-rows 80 bytes
//   apart, so that the four lane groups of a read fall on different banks).
//   Reading such an operand 2 bytes per lane along its columns instead took
//   three times as long (a quarter of each 128-byte line per load, and eight
//   loads per fragment).
// Columns of B are assigned to workgroups so that the eight XCDs each take one
// contiguous range: the 16-column blocks that share a 128-byte line of a
// row-major B then share one XCD's L2.
//
// The same kernel takes the last few columns of a product as the transposed
// product C^T = B^T A^T (M and N swapped, B's column slab as the left operand,
// A as the right one), writing element (i, j) to C[j * ldc + i] (trans_c): a
// lane's four rows of a 16 x 16 block are then four consecutive elements of
// one row of C.
//
// Requirements (the launcher returns hipErrorInvalidValue otherwise): operands
// 16-byte aligned with leading dimensions in whole 16-byte chunks, and K in
// whole chunks for a k-contiguous operand (or the operand a copy zero-filled to
// one), so that its chunks along k are wholly inside the matrix or wholly past
// K.  The side of an operand with k as its row index (N of row-major B, M of A
// given transposed) may end inside a chunk.
#include "mfma16_direct.hpp"

namespace migemm {
namespace {

// Sixteen waves of five k-steps per round when A is k-contiguous; eight of four
// when A is given transposed, where both operands may be staged through LDS.
template <typename E, bool TA, bool TB> struct Shape {
    static constexpr int kWaves = TA ? 8 : 16, kBatch = TA ? 4 : 5;
    static constexpr int EPC = 16 / sizeof(E);     // elements per 16-byte chunk
    static constexpr int KSTEP = 4 * EPC;          // k per step: four lane groups
    static constexpr int CPR = 16 / EPC;           // chunks per 16-column k-row
    static constexpr int ROW_BYTES = EPC == 16 ? 16 : EPC == 8 ? 32 : 80;  // a k-row in an LDS slot
    static constexpr int SLOT = KSTEP * ROW_BYTES;  // 1 KiB (8- and 16-bit), 1280 B (FP32)
    static constexpr int kRowOps = (TA ? 1 : 0) + (TB ? 0 : 1);  // operands with k as row index
    static constexpr int kSlots = kRowOps ? kBatch * kRowOps : 1;
};

// The 16-byte k-run [k0, k0 + EPC) of row `row` of a k-contiguous operand.
template <typename E>
__device__ __forceinline__ u32x4 krun(const E* __restrict__ p, int64_t ld, int64_t row,
                                      int64_t k0) {
    return *reinterpret_cast<const u32x4*>(p + row * ld + k0);
}

// This lane's 16-byte chunk of k-step s of an operand stored with k as its row
// index (cols columns, this workgroup's 16 starting at c0): k-row
// KSTEP s + lane / CPR, columns c0 + EPC (lane % CPR) onwards; zeros past K or
// past cols.  A chunk that cols ends inside is read as its valid bytes only, in
// at most four naturally aligned pieces (8, 4, 2 and 1 bytes, the chunk being
// 16-byte aligned), so no byte past the matrix is touched.
template <typename E, int KSTEP, int EPC>
__device__ __forceinline__ u32x4 krow_chunk(const E* __restrict__ p, int64_t ld, int64_t cols,
                                            int64_t c0, int64_t K, int64_t s, int lane) {
    constexpr int CPR = 16 / EPC;
    const int64_t kr = KSTEP * s + lane / CPR, c = c0 + EPC * (lane % CPR);
    if (kr >= K || c >= cols) return u32x4{0u, 0u, 0u, 0u};
    const E* q = p + kr * ld + c;
    if (c + EPC <= cols) return *reinterpret_cast<const u32x4*>(q);
    const int nb = static_cast<int>(cols - c) * static_cast<int>(sizeof(E));  // 1 .. 15 bytes
    const unsigned char* qb = reinterpret_cast<const unsigned char*>(q);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (nb & 8) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(qb);
        v[0] = x[0];
        v[1] = x[1];
    }
    const int o4 = nb & 8;  // offsets of the 4-, 2- and 1-byte pieces
    const int o2 = o4 + (nb & 4), o1 = o2 + (nb & 2);
    uint32_t w4 = 0u, w2 = 0u, w1 = 0u;
    if (nb & 4) w4 = *reinterpret_cast<const uint32_t*>(qb + o4);
    if (nb & 2) w2 = *reinterpret_cast<const uint16_t*>(qb + o2);
    if (nb & 1) w1 = static_cast<uint32_t>(qb[o1]) << (8 * (o1 % 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // dword j collects the pieces that start in it (the 2-byte piece starts
        // on a dword, the 1-byte piece anywhere)
        v[j] |= (o4 / 4 == j && (nb & 4) ? w4 : 0u) | (o2 / 4 == j ? w2 : 0u) |
                (o1 / 4 == j ? w1 : 0u);
    }
    return v;
}

// Stages a step's k-rows x 16 columns (lane l's chunk: k-row l / CPR, chunk
// l % CPR) in this wave's slot and returns the fragment of lane (r, g) =
// (lane % 16, lane / 16): column r of k-rows EPC g .. EPC g + EPC - 1.  The
// wave's LDS operations run in order, so the reads see the write without a
// barrier.
template <int EPC>
__device__ __forceinline__ u32x4 stage_krow(MIGEMM_LDS char* slot, u32x4 chunk, int lane) {
    const int r = lane % 16, g = lane / 16;
    if constexpr (EPC == 16) {
        // 16-byte k-rows, one per lane.  In each 16-lane group, lanes 2 i and
        // 2 i + 1 address the two 8-byte halves of k-row 16 g + i (+ 8 for the
        // second read), and the transposing read returns column r of those eight
        // k-rows to lane r.
        *(MIGEMM_LDS u32x4*)(slot + 16 * lane) = chunk;
        MIGEMM_LDS char* p = slot + (16 * g + r / 2) * 16 + 8 * (r % 2);
        const u32x2 lo = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((MIGEMM_LDS i32x2*)p));
        const u32x2 hi = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((MIGEMM_LDS i32x2*)(p + 8 * 16)));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else if constexpr (EPC == 8) {
        // 32-byte k-rows.  In each 16-lane group, lanes 4 i .. 4 i + 3 address
        // the four 8-byte pieces of k-row 8 g + i (+ 4 for the second read), and
        // the transposing read returns column r of those four k-rows to lane r.
        *(MIGEMM_LDS u32x4*)(slot + 16 * lane) = chunk;
        MIGEMM_LDS char* p = slot + (8 * g + r / 4) * 32 + 8 * (r % 4);
        const u32x2 lo = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIGEMM_LDS s16x4*)p));
        const u32x2 hi = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIGEMM_LDS s16x4*)(p + 4 * 32)));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else {
        // 80-byte k-rows (64 bytes of data): a read of k-row 4 g + e by the four
        // lane groups touches dwords 80 (4 g + e) / 4 + r, i.e. banks
        // 16 g + 20 e + r (mod 64): four disjoint runs of 16.
        *(MIGEMM_LDS u32x4*)(slot + (lane / 4) * 80 + 16 * (lane % 4)) = chunk;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = *(const MIGEMM_LDS uint32_t*)(slot + (4 * g + e) * 80 + 4 * r);
        return v;
    }
}

// TA: A stored K x M; TB: B stored N x K (k contiguous); TC: C written
// transposed.
template <typename E, bool GEN, bool TA, bool TB, bool TC>
__global__ __launch_bounds__((Shape<E, TA, TB>::kWaves * kWave)) void skinny_kernel(
    int64_t M, int64_t N, int64_t K, const E* __restrict__ A, int64_t lda,
    const E* __restrict__ B, int64_t ldb, Epi out) {
    using Op = MfmaOp<E, 16>;
    using Acc = typename Op::Acc;  // f32x4, or i32x4 for INT8
    using L = AccLayout<16>;
    using Sh = Shape<E, TA, TB>;
    constexpr int kWaves = Sh::kWaves, kBatch = Sh::kBatch, EPC = Sh::EPC, KSTEP = Sh::KSTEP;
    __shared__ Acc part[kWaves][kWave];
    __shared__ __attribute__((aligned(16))) char stage[Sh::kRowOps ? kWaves : 1][Sh::kSlots * Sh::SLOT];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int r = lane % 16, g = lane / 16;
    // column block: XCD x (blockIdx modulo 8) takes one contiguous range
    const int64_t per = gridDim.x / kNumXcd;
    const int64_t blk = blockIdx.x < per * kNumXcd
                            ? (blockIdx.x % kNumXcd) * per + blockIdx.x / kNumXcd
                            : blockIdx.x;
    const int64_t n0 = blk * 16;
    const int64_t n = min(n0 + r, N - 1);  // B column fed by this lane (clamped; k-contiguous B)
    const bool a_in = r < M;
    MIGEMM_LDS char* const slots =
        (MIGEMM_LDS char*)&stage[0][0] + (Sh::kRowOps ? wave : 0) * (Sh::kSlots * Sh::SLOT);
    Acc acc = {};
    const int64_t steps = ceil_div(K, KSTEP);
    // kBatch of this wave's steps per round, all their loads issued before the
    // first matrix instruction: one memory latency per round instead of per step
    for (int64_t s0 = wave; s0 < steps; s0 += kBatch * kWaves) {
        u32x4 a[kBatch], b[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int64_t s = s0 + q * kWaves;
            a[q] = b[q] = u32x4{0u, 0u, 0u, 0u};
            if (s < steps) {
                const int64_t k0 = s * KSTEP + EPC * g;
                if constexpr (TA)
                    a[q] = krow_chunk<E, KSTEP, EPC>(A, lda, M, 0, K, s, lane);
                else if (a_in && k0 < K)
                    a[q] = krun(A, lda, r, k0);
                if constexpr (TB) {
                    if (k0 < K) b[q] = krun(B, ldb, n, k0);
                } else {
                    b[q] = krow_chunk<E, KSTEP, EPC>(B, ldb, N, n0, K, s, lane);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            MIGEMM_LDS char* const slot = slots + q * Sh::kRowOps * Sh::SLOT;
            if constexpr (TA) a[q] = stage_krow<EPC>(slot, a[q], lane);
            if constexpr (!TB) b[q] = stage_krow<EPC>(slot + (TA ? Sh::SLOT : 0), b[q], lane);
            Op::run(acc, a[q], b[q]);
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    Acc sum = part[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        const Acc p = part[w][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[e] += p[e];
    }
    const int64_t col = n0 + L::col(lane);
    if (col >= N) return;
#pragma unroll
    for (int e = 0; e < L::R; ++e) {
        const int64_t row = L::row(lane, e);
        if (row >= M) continue;
        const int64_t idx = TC ? col * out.ldc + row : row * out.ldc + col;
        if constexpr (sizeof(E) == 1)
            static_cast<int32_t*>(out.C)[idx] = sum[e];  // exact INT32 sums
        else
            store_out<GEN>(out, idx, sum[e]);
    }
}

template <typename E, bool GEN, bool TC>
hipError_t launch_typed(const GemmArgs& g) {
    const dim3 grid(static_cast<unsigned>(ceil_div(g.N, 16)));
    const E* A = static_cast<const E*>(g.A);
    const E* B = static_cast<const E*>(g.B);
#define MIGEMM_LAUNCH(TA_, TB_)                                                                \
    return launch_kernel(g, skinny_kernel<E, GEN, TA_, TB_, TC>, grid,                        \
                         dim3(Shape<E, TA_, TB_>::kWaves * kWave), g.M, g.N, g.K, A, g.lda, B, \
                         g.ldb, g.out)
    if (g.ta) {
        if (g.tb) MIGEMM_LAUNCH(true, true);
        MIGEMM_LAUNCH(true, false);
    }
    if (g.tb) MIGEMM_LAUNCH(false, true);
    MIGEMM_LAUNCH(false, false);
#undef MIGEMM_LAUNCH
}

template <typename E, bool GEN>
hipError_t launch_out(const GemmArgs& g) {
    return g.trans_c ? launch_typed<E, GEN, true>(g) : launch_typed<E, GEN, false>(g);
}

template <typename E>
hipError_t launch_elem(const GemmArgs& g) {
    return g.general() ? launch_out<E, true>(g) : launch_out<E, false>(g);
}

}  // namespace

bool skinny_fits(const GemmArgs& g) {
    if (g.dtype != 0 && g.dtype != 1 && g.dtype != 2 && g.dtype != 3) return false;
    if (g.dtype == 3 && g.out.c_dtype != 4) return false;  // INT8: INT32 C only
    // every operand is read in aligned 16-byte chunks: a k-contiguous one in
    // whole chunks of k (unless it is a zero-filled copy); one with k as its row
    // index reads a last partial chunk of its columns element by element
    const int64_t epc = g.dtype == 0 ? 4 : g.dtype == 3 ? 16 : 8;
    const bool k_whole = g.K % epc == 0;
    const bool a_ok = aligned16(g.A) && g.lda % epc == 0 && (g.ta || k_whole || g.pad_a);
    const bool b_ok = aligned16(g.B) && g.ldb % epc == 0 && (!g.tb || k_whole || g.pad_b);
    return g.M >= 1 && g.M <= 16 && g.N >= 1 && g.K > 0 && a_ok && b_ok &&
           ceil_div(g.N, 16) <= 0x7fffffff;
}

hipError_t launch_skinny(const GemmArgs& g) {
    if (!skinny_fits(g)) return hipErrorInvalidValue;
    if (g.dtype == 0) return launch_elem<float>(g);
    if (g.dtype == 3) return launch_out<int8_t, false>(g);  // INT32 C, plain overwrite
    return g.dtype == 1 ? launch_elem<_Float16>(g) : launch_elem<bf16_t>(g);
}

}  // namespace migemm
