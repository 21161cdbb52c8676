// mfma_gemm.hpp -- the LDS-staged matrix-core GEMM pipeline for gfx950.
//
// Algorithm (page "Tensor cores and matrix operations", section "Complete
// Algorithm for Large Matrix Multiply"): C is cut into output tiles, each
// tile's accumulator starts at zero, and the inner dimension is walked in
// k-tiles; every k-tile contributes the product of an A tile and a B tile,
// evaluated as a grid of small matrix-unit products that all add into the
// tile's accumulator.  Because the partial products simply add, the order of
// the k-tiles does not change the result beyond FP32 rounding.
//
// What changes for gfx950 (instead of the pages' 16x16x16 warp fragments
// loaded straight from global memory, page "CUDA-Practice 09", section on
// the naive WMMA kernel, where the matrix units wait on memory):
//
// * Staging.  A workgroup tile BM x BN is built from k-tiles of 128 bytes per
//   row (BK = 64 FP16/BF16 or 32 FP32 elements).  Global memory is read with
//   16-byte vector loads into registers, the next k-tile's loads are issued
//   before the current k-tile's matrix work, and the registers are written to
//   the other half of a double-buffered LDS tile afterwards: one barrier per
//   k-tile.
// * Operand layout.  A matrix-core instruction wants, in every lane, a run of
//   consecutive k for one row of A and for one column of B.  An operand stored
//   with k contiguous (row-major A, or B given transposed) is copied in 16-byte
//   chunks along k.  One stored with its M or N side contiguous (row-major B, or
//   A given transposed) is loaded in VEC x VEC blocks (VEC rows of k, one
//   16-byte chunk across) and transposed in registers before the LDS write.
//   Either way both operands sit in LDS as [row][k] with 16-byte chunks, and
//   every fragment read is one 16-byte LDS read per lane.
// * Bank conflicts.  Rows are 128 bytes long, so without care every row of a
//   fragment read would hit the same banks.  The chunk index is XOR-swizzled
//   with (row ^ (row >> 3)) & 7: sixteen consecutive rows reading the same
//   logical chunk then touch sixteen distinct 16-byte bank groups, and the
//   transposed B writes (rows 8 apart) are spread the same way.
// * Matrix instructions.  Lanes are split into G = 64 / MF groups; lane
//   (r + MF * g) holds row r of its MF-row block and chunk g of a k-slab of G
//   chunks.  A and B use the same lane-to-k assignment, so the instruction's
//   sum over k pairs the right elements whatever order it adds them in.
//   FP16/BF16: one v_mfma_f32_{16x16x32,32x32x16} per slab consumes one chunk
//   per lane; FP32: four v_mfma_f32_{16x16x4,32x32x2}_f32, one per element.
// * Tile order.  Workgroups are dealt round-robin to the 8 XCDs, each with its
//   own L2.  Workgroup ids are remapped so that each XCD receives a
//   contiguous range of tiles, and tiles are ordered in bands of GM tile-rows,
//   so the tiles resident on one XCD share rows of A and columns of B.
// * Edges.  Any M, N, K and leading dimension is accepted.  Tiles that lie
//   fully inside the matrix and k-tiles that lie fully inside K take the
//   unguarded vector path; the others load zeros for out-of-range elements
//   and store only in-range outputs.  Operands whose rows are not 16-byte
//   aligned are read element by element.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace migemm {

template <typename E> struct Elem;
template <> struct Elem<float> { static constexpr int VEC = 4; };     // elements per 16 bytes
template <> struct Elem<_Float16> { static constexpr int VEC = 8; };
template <> struct Elem<bf16_t> { static constexpr int VEC = 8; };
template <> struct Elem<int8_t> { static constexpr int VEC = 16; };

// One matrix-core step consuming one 16-byte chunk of A and of B in each lane.
template <typename E, int MF> struct MfmaOp;

template <> struct MfmaOp<bf16_t, 16> {
    using Acc = f32x4;
    static __device__ __forceinline__ void run(Acc& c, u32x4 a, u32x4 b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct MfmaOp<bf16_t, 32> {
    using Acc = f32x16;
    static __device__ __forceinline__ void run(Acc& c, u32x4 a, u32x4 b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct MfmaOp<_Float16, 16> {
    using Acc = f32x4;
    static __device__ __forceinline__ void run(Acc& c, u32x4 a, u32x4 b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <> struct MfmaOp<_Float16, 32> {
    using Acc = f32x16;
    static __device__ __forceinline__ void run(Acc& c, u32x4 a, u32x4 b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <> struct MfmaOp<float, 16> {
    using Acc = f32x4;
    static __device__ __forceinline__ void run(Acc& c, u32x4 a, u32x4 b) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]),
                                                     c, 0, 0, 0);
    }
};
template <> struct MfmaOp<float, 32> {
    using Acc = f32x16;
    static __device__ __forceinline__ void run(Acc& c, u32x4 a, u32x4 b) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]),
                                                     c, 0, 0, 0);
    }
};

// INT8: one instruction per 16-byte chunk (16 k per lane), exact INT32 sums.
template <> struct MfmaOp<int8_t, 16> {
    using Acc = i32x4;
    static __device__ __forceinline__ void run(Acc& c, u32x4 a, u32x4 b) {
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                  __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
};
template <> struct MfmaOp<int8_t, 32> {
    using Acc = i32x16;
    static __device__ __forceinline__ void run(Acc& c, u32x4 a, u32x4 b) {
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                  __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
};

// Accumulator element r of lane `lane` in an MF x MF block: (row, col) in the block.
template <int MF> struct AccLayout;
template <> struct AccLayout<16> {  // 4 rows per lane: rows 4g..4g+3 of column lane % 16
    static constexpr int R = 4;
    static __device__ __forceinline__ int row(int lane, int r) { return 4 * (lane >> 4) + r; }
    static __device__ __forceinline__ int col(int lane) { return lane & 15; }
};
template <> struct AccLayout<32> {  // 16 values per lane in 4 runs of 4 rows, 8 rows apart
    static constexpr int R = 16;
    static __device__ __forceinline__ int row(int lane, int r) {
        return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    }
    static __device__ __forceinline__ int col(int lane) { return lane & 31; }
};

// Physical 16-byte chunk of logical chunk c in LDS row `row` (8 chunks per row).
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

// Element type used for guarded scalar loads.
template <typename E> struct Scalar { using T = E; };
template <> struct Scalar<bf16_t> { using T = uint16_t; };
template <> struct Scalar<_Float16> { using T = uint16_t; };
template <> struct Scalar<float> { using T = uint32_t; };
template <> struct Scalar<int8_t> { using T = uint8_t; };

// Loads the 16-byte chunk of VEC elements at (r, c0 .. c0+VEC-1) of a row-major
// nrows x ncols matrix; out-of-range elements read as zero.
template <typename E, bool VECOK>
__device__ __forceinline__ u32x4 load_chunk_guarded(const E* __restrict__ base, int64_t r,
                                                    int64_t c0, int64_t nrows, int64_t ncols,
                                                    int64_t ld) {
    constexpr int VEC = Elem<E>::VEC;
    using S = typename Scalar<E>::T;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r >= nrows) return v;
    const E* p = base + r * ld + c0;
    if (VECOK && c0 + VEC <= ncols) return *reinterpret_cast<const u32x4*>(p);
    const S* ps = reinterpret_cast<const S*>(p);
    if constexpr (sizeof(S) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (c0 + e < ncols) ? ps[e] : 0u;
    } else if constexpr (sizeof(S) == 1) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (c0 + e < ncols) v[e / 4] |= static_cast<uint32_t>(ps[e]) << (8 * (e % 4));
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = (c0 + 2 * e < ncols) ? ps[2 * e] : 0u;
            const uint32_t hi = (c0 + 2 * e + 1 < ncols) ? ps[2 * e + 1] : 0u;
            v[e] = lo | (hi << 16);
        }
    }
    return v;
}

// Transposes a VEC x VEC block held as VEC row chunks into VEC column chunks.
template <int VEC> struct Transpose;
template <> struct Transpose<8> {  // 16-bit elements: dword d of a row holds columns 2d, 2d+1
    static __device__ __forceinline__ void run(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = in[2 * e][c >> 1], hi = in[2 * e + 1][c >> 1];
                out[c][e] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                    : ((lo & 0xffffu) | (hi << 16));
            }
        }
    }
};
template <> struct Transpose<4> {  // 32-bit elements
    static __device__ __forceinline__ void run(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) out[c][e] = in[e][c];
    }
};

// Workgroup `bid` of `total` renumbered so that each XCD (bid modulo 8, the
// round-robin order in which workgroups are dealt to the XCDs) takes one
// contiguous range of the new numbers; the last total mod 8 keep theirs.
__device__ __forceinline__ int xcd_contiguous(int bid, int total) {
    const int per = total / kNumXcd;
    return bid < per * kNumXcd ? (bid % kNumXcd) * per + bid / kNumXcd : bid;
}

// Tile (pm, pn) number `id` in GM-row bands: GM tile rows at a time, down the
// rows of a band, then across its columns.
template <int GM>
__device__ __forceinline__ void band_coords(int id, int tiles_m, int tiles_n, int& pm, int& pn) {
    const int band = GM * tiles_n;
    const int first_m = (id / band) * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in = id % band;
    pm = first_m + in % gm;
    pn = in / gm;
}

// Tile (pm, pn) processed by workgroup `bid`: XCD-contiguous ranges, GM-row bands.
template <int GM>
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& pm, int& pn) {
    band_coords<GM>(xcd_contiguous(bid, tiles_m * tiles_n), tiles_m, tiles_n, pm, pn);
}

// One operand's staging: a BX x BK tile (BX rows of M or N, BK of k) from global
// memory through registers into a swizzled [row][k] LDS image.  KC: the operand
// is stored with k contiguous; otherwise with the BX side contiguous (loaded in
// VEC x VEC blocks and transposed in registers).  VECOK: rows are 16-byte
// aligned, so in-range chunks take one vector load.
//
// 8-bit elements (VEC = 16) not k-contiguous are staged in quarter blocks: a
// work-item loads 4 k-rows of one 16-byte piece, transposes them as four 4 x 4
// byte blocks and writes 4-byte column pieces, so every work-item takes one
// quarter instead of a quarter of the work-items taking whole 16 x 16 blocks.
template <typename E, int BX, int NT, bool KC, bool VECOK>
struct Stage {
    static constexpr int VEC = Elem<E>::VEC, CH = 8;
    static constexpr bool QUARTER = !KC && VEC == 16;
    static constexpr int ROWS = KC ? 1 : QUARTER ? 4 : VEC;  // rows per staging unit
    // chunks, VEC x VEC blocks, or quarter blocks
    static constexpr int UNITS = KC ? BX * CH : QUARTER ? CH * (BX / VEC) * 4 : CH * (BX / VEC);
    static constexpr int PER = (UNITS + NT - 1) / NT;
    static_assert(BX % VEC == 0, "tile side must be whole chunks");
    u32x4 r[PER][ROWS];

    // Tile rows x0 .. x0+BX-1 (of ext) and k0 .. k0+BK-1 (of K); p and ld as stored.
    // fast: the tile lies inside the matrix, no guards needed.
    __device__ __forceinline__ void load(const E* __restrict__ p, int64_t ld, int tid, int64_t x0,
                                         int64_t k0, int64_t ext, int64_t K, bool fast) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int id = tid + q * NT;
            if (UNITS % NT != 0 && id >= UNITS) continue;
            if constexpr (KC) {
                const int64_t gr = x0 + id / CH, gc = k0 + (id % CH) * VEC;
                r[q][0] = (VECOK && fast) ? *reinterpret_cast<const u32x4*>(p + gr * ld + gc)
                                          : load_chunk_guarded<E, VECOK>(p, gr, gc, ext, K, ld);
            } else if constexpr (QUARTER) {
                // id -> piece across the row (fastest, for coalescing), quarter, k-block
                const int xb = id % (BX / VEC), qq = (id / (BX / VEC)) % 4;
                const int kb = id / (BX / VEC) / 4;
                const int64_t gc = x0 + xb * VEC;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t gr = k0 + kb * VEC + 4 * qq + e;
                    r[q][e] = (VECOK && fast) ? *reinterpret_cast<const u32x4*>(p + gr * ld + gc)
                                              : load_chunk_guarded<E, VECOK>(p, gr, gc, K, ext, ld);
                }
            } else {
                const int64_t gc = x0 + (id % (BX / VEC)) * VEC;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int64_t gr = k0 + (id / (BX / VEC)) * VEC + e;
                    r[q][e] = (VECOK && fast) ? *reinterpret_cast<const u32x4*>(p + gr * ld + gc)
                                              : load_chunk_guarded<E, VECOK>(p, gr, gc, K, ext, ld);
                }
            }
        }
    }

    // Registers -> LDS image `img` ([BX rows][CH chunks], chunks swizzled per row).
    __device__ __forceinline__ void store(u32x4* img, int tid) const {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int id = tid + q * NT;
            if (UNITS % NT != 0 && id >= UNITS) continue;
            if constexpr (KC) {
                const int row = id / CH, ch = id % CH;
                img[row * CH + swz(row, ch)] = r[q][0];
            } else if constexpr (QUARTER) {
                const int xb = id % (BX / VEC), qq = (id / (BX / VEC)) % 4;
                const int kb = id / (BX / VEC) / 4;
                uint32_t* words = reinterpret_cast<uint32_t*>(img);
#pragma unroll
                for (int cw = 0; cw < 4; ++cw) {
                    // 4 x 4 bytes: k-rows 4qq .. 4qq+3 of columns 16 xb + 4 cw .. + 3
                    const uint32_t r0 = r[q][0][cw], r1 = r[q][1][cw];
                    const uint32_t r2 = r[q][2][cw], r3 = r[q][3][cw];
                    const uint32_t t0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
                    const uint32_t t1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
                    const uint32_t t2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
                    const uint32_t t3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
                    const uint32_t col[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u),
                                             __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                                             __builtin_amdgcn_perm(t3, t1, 0x05040100u),
                                             __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int row = xb * VEC + 4 * cw + j;
                        words[(row * CH + swz(row, kb)) * 4 + qq] = col[j];
                    }
                }
            } else {
                const int xb = id % (BX / VEC), kb = id / (BX / VEC);
                u32x4 t[VEC];
                Transpose<VEC>::run(r[q], t);
#pragma unroll
                for (int c = 0; c < VEC; ++c) {
                    const int row = xb * VEC + c;
                    img[row * CH + swz(row, kb)] = t[c];
                }
            }
        }
    }
};

template <typename E_, int BM_, int BN_, int WM_, int WN_, int MF_, int GM_ = 8>
struct MfmaCfg {
    using E = E_;
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MF = MF_, GM = GM_;
    static constexpr int NT = WM * WN * kWave;
    static constexpr int VEC = Elem<E>::VEC;
    static constexpr int CH = 8;  // 16-byte chunks per LDS row: 128 bytes of k
    static constexpr int BK = CH * VEC;
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    static constexpr int TM = WTM / MF, TN = WTN / MF;  // matrix-core blocks per wave
    static constexpr int G = kWave / MF;                // lane groups
    static constexpr int SLABS = CH / G;                // k-slabs per k-tile
    static constexpr int LDS_BYTES = 2 * (BM + BN) * CH * 16;
    static_assert(BM % (WM * MF) == 0 && BN % (WN * MF) == 0, "wave tiles must be whole blocks");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS is 160 KiB per CU on gfx950");
    static_assert(NT <= 1024, "at most 1024 work-items per workgroup");
};

// TA: A is given transposed (stored K x M, m contiguous); TB: B is given
// transposed (stored N x K, k contiguous).
template <class Cfg, bool AV, bool BV, bool GEN, bool TA, bool TB>
__global__ __launch_bounds__(Cfg::NT) void mfma_gemm_kernel(
    int64_t M, int64_t N, int64_t K, const typename Cfg::E* __restrict__ A, int64_t lda,
    const typename Cfg::E* __restrict__ B, int64_t ldb, Epi out, int tiles_m, int tiles_n) {
    using E = typename Cfg::E;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, MF = Cfg::MF, NT = Cfg::NT;
    constexpr int CH = Cfg::CH, BK = Cfg::BK, TM = Cfg::TM, TN = Cfg::TN, G = Cfg::G;
    using Op = MfmaOp<E, MF>;
    using Acc = typename Op::Acc;
    using L = AccLayout<MF>;

    __shared__ u32x4 sA[2][BM * CH];
    __shared__ u32x4 sB[2][BN * CH];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm0 = (wave / Cfg::WN) * Cfg::WTM;
    const int wn0 = (wave % Cfg::WN) * Cfg::WTN;

    int pm, pn;
    tile_coords<Cfg::GM>(blockIdx.x, tiles_m, tiles_n, pm, pn);
    const int64_t m0 = static_cast<int64_t>(pm) * BM;
    const int64_t n0 = static_cast<int64_t>(pn) * BN;
    const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Acc{};

    // A is k-contiguous unless given transposed; B only when given transposed.
    Stage<E, BM, NT, !TA, AV> stA;
    Stage<E, BN, NT, TB, BV> stB;

    // Global -> registers for k-tile kt.
    auto load_tile = [&](int kt) {
        const int64_t k0 = static_cast<int64_t>(kt) * BK;
        const bool fast = full_mn && (k0 + BK <= K);
        stA.load(A, lda, tid, m0, k0, M, K, fast);
        stB.load(B, ldb, tid, n0, k0, N, K, fast);
    };

    // Registers -> LDS buffer `buf`, both operands as [row][k].
    auto store_tile = [&](int buf) {
        stA.store(sA[buf], tid);
        stB.store(sB[buf], tid);
    };

    const int KT = static_cast<int>(ceil_div(K, BK));
    if (KT > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    const int lr = lane % MF;  // row (or column) of the block this lane feeds
    const int lg = lane / MF;  // chunk group this lane feeds
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_tile(kt + 1);
#pragma unroll
        for (int s = 0; s < Cfg::SLABS; ++s) {
            const int ch = s * G + lg;
            u32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm0 + i * MF + lr;
                fa[i] = sA[cur][row * CH + swz(row, ch)];
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn0 + j * MF + lr;
                fb[j] = sB[cur][row * CH + swz(row, ch)];
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) Op::run(acc[i][j], fa[i], fb[j]);
        }
        if (kt + 1 < KT) store_tile(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: FP32 accumulators -> C through the output step.
    const int lc = L::col(lane);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wn0 + j * MF + lc;
#pragma unroll
            for (int r = 0; r < L::R; ++r) {
                const int64_t row = m0 + wm0 + i * MF + L::row(lane, r);
                if (full_mn || (row < M && col < N)) {
                    if constexpr (std::is_same<E, int8_t>::value)  // exact INT32 sums
                        static_cast<int32_t*>(out.C)[row * out.ldc + col] = acc[i][j][r];
                    else
                        store_out<GEN>(out, row * out.ldc + col, acc[i][j][r]);
                }
            }
        }
    }
}

// Host side: launches configuration Cfg on the given arguments, with the
// plain FP32 overwrite (GEN == false) or the general output step.
template <class Cfg, bool GEN>
hipError_t launch_mfma_cfg(const GemmArgs& g) {
    if (g.splitk > 1) return hipErrorInvalidValue;  // split-K runs on the direct kernel only
    using E = typename Cfg::E;
    constexpr int VEC = Cfg::VEC;
    const int64_t tm = ceil_div(g.M, Cfg::BM), tn = ceil_div(g.N, Cfg::BN);
    if (tm * tn > 0x7fffffff) return hipErrorInvalidValue;
    const bool av = aligned16(g.A) && (g.lda % VEC) == 0;
    const bool bv = aligned16(g.B) && (g.ldb % VEC) == 0;
    const E* A = static_cast<const E*>(g.A);
    const E* B = static_cast<const E*>(g.B);
    dim3 grid(static_cast<unsigned>(tm * tn)), block(Cfg::NT);
    const int itm = static_cast<int>(tm), itn = static_cast<int>(tn);
    // The plain row-major product is compiled for all four load forms; the
    // general output step and the transposed layouts for the two common ones
    // (both operands vectorised, or neither), which bounds the instantiations.
#define MIGEMM_LAUNCH(AV_, BV_, TA_, TB_)                                                      \
    return launch_kernel(g, mfma_gemm_kernel<Cfg, AV_, BV_, GEN, TA_, TB_>, grid, block, g.M,   \
                         g.N, g.K, A, g.lda, B, g.ldb, g.out, itm, itn)
    const bool vec = av && bv;
    if (g.ta || g.tb) {
        if (g.ta && g.tb) {
            if (vec) MIGEMM_LAUNCH(true, true, true, true); else MIGEMM_LAUNCH(false, false, true, true);
        } else if (g.ta) {
            if (vec) MIGEMM_LAUNCH(true, true, true, false); else MIGEMM_LAUNCH(false, false, true, false);
        } else {
            if (vec) MIGEMM_LAUNCH(true, true, false, true); else MIGEMM_LAUNCH(false, false, false, true);
        }
    } else if (GEN || vec) {
        if (vec) MIGEMM_LAUNCH(true, true, false, false); else MIGEMM_LAUNCH(false, false, false, false);
    } else if (av) {
        MIGEMM_LAUNCH(true, false, false, false);
    } else if (bv) {
        MIGEMM_LAUNCH(false, true, false, false);
    } else {
        MIGEMM_LAUNCH(false, false, false, false);
    }
#undef MIGEMM_LAUNCH
}

}  // namespace migemm
