// mfma16_direct.hpp -- FP16/BF16 (and INT8) GEMM for gfx950 with direct
// global->LDS staging and transposing LDS reads.
//
// Same algorithm as mfma_gemm.hpp (tiles of C, k-tiles accumulated by the
// matrix cores; page "Tensor cores and matrix operations", section "Complete
// Algorithm for Large Matrix Multiply"), rebuilt around two gfx950 features:
//
// * global_load_lds_dwordx4 moves 16 bytes per lane from global memory
//   straight into LDS (lane l's bytes land at the instruction's LDS base +
//   16 l), so no registers hold staged tiles and no instructions copy them.
//   Which global chunk a lane fetches is chosen so that the LDS image comes out
//   swizzled.
// * ds_read_b64_tr_b16 reads a 4-row x 16-column block of a row-major tile and
//   hands lane j of each 16-lane group column j of those rows (ds_read_b64_tr_b8:
//   an 8-row x 16-byte block, for 8-bit elements).  B therefore stays row-major
//   in LDS (as it is in memory), and the k-contiguous operand the matrix
//   instruction wants is produced by the read itself: two transposing reads
//   give a lane the 16 bytes of consecutive k of one column of B.
//
// Everything is counted in 16-byte chunks, so the code serves 4-, 2- and
// 1-byte elements alike: a 32-deep FP32 k-tile, a 64-deep 16-bit one and a
// 128-deep 8-bit one are all 128 bytes per row.
//
// FP32 (v_mfma_f32_16x16x4_f32, one element per lane and instruction): a 16-byte
// row-image read hands a lane four consecutive k of one row of A, which feed
// four instructions (element e to instruction e).  The matching B values are
// four k-rows of one column; a k-row image has no 32-bit transposing read, so
// they come from four 4-byte LDS reads, one per k-row.  The k-row swizzle
// (swz_b32) puts the four lane groups of such a read on four distinct 16-bank
// quarters.
//
// LDS images (per stage):
//   A: [BM rows][8 chunks of 16 B]; logical chunk c of row r at physical chunk
//      c ^ ((r >> 1) & 7).  Sixteen consecutive rows reading one logical chunk
//      (a fragment read) then fall on sixteen distinct 16-byte bank groups: the
//      eight even rows on one half of the banks, the eight odd rows on the other,
//      each on its own chunk.  The pattern repeats every 16 rows, so fragments
//      16 rows apart differ by a constant address offset.
//   B: [k-rows][BN elements]; logical chunk c of k-row r at c ^ swizzle(r):
//      16-bit, BN >= 128: 2 f(r), f(r) = (r & 3) | (((r >> 3) & 1) << 2).  A
//      transposing read touches 32 bytes (two chunks) in each of the rows
//      8g + {0..3} of the four lane groups g; f gives the eight rows of two
//      adjacent groups eight distinct chunk pairs, i.e. all 64 banks once.
//      16-bit, BN = 64, and 8-bit: see swz_b64 and swz_b8 below.
//
// Work per workgroup: a BM x BN tile of C, WM x WN wavefronts each owning a
// (BM/WM) x (BN/WN) block of accumulators.  Two schedules:
// * interleaved (SCHED 0 or 2): k advances one k-tile at a time through
//   STAGES LDS buffers; the direct loads of k-tile kt + STAGES - 1 are issued
//   at the start of k-tile kt (or, with early loads, right after the barrier
//   that frees their stage), and the fragments of the next slab are read from
//   LDS while the current slab's instructions run, including across the one
//   barrier per k-tile;
// * ping-pong (SCHED 4, whole tiles only): two groups of four waves take
//   turns on each SIMD, one running a whole k-tile of matrix instructions
//   while the other reads its next k-tile of fragments and issues direct
//   loads (see the kernel body).
//
// The direct loads are issued through inline assembly with explicit
// vmcnt accounting: the compiler cannot see that they write a different LDS
// stage from the one being read, and would otherwise wait for every load
// before every LDS read.  They use an SGPR tile base plus a 32-bit per-lane
// offset, so the per-lane offsets are computed once and no 64-bit addresses
// occupy VGPRs.
//
// Operands given transposed swap image kinds: A stored K x M (m contiguous)
// becomes a k-row image like B's and is read with transposing reads; B stored
// N x K (k contiguous) becomes a row image like A's and is read with
// ds_read_b128.  Both reads hand a lane the same fragment (a 16-byte run of k
// of one row of A or column of B), so the matrix instructions do not change.
//
// Preconditions (checked by the launcher; other shapes use mfma_gemm.hpp):
// A and B 16-byte aligned, lda and ldb in whole 16-byte chunks, K in whole
// chunks (a multiple of the k-tile without flag bit 5), and the side of a k-row
// image (N for row-major B, M for A given transposed) in whole chunks; the
// ping-pong schedule also needs M and N to be multiples of the tile.  Rows of a row image
// past M or N, and chunks of a k-row image past its side, are clamped to the
// last valid row / chunk, so every load is in bounds; those lanes only feed
// outputs that are never stored.  A last k-tile that K ends inside is loaded
// with its chunks (row image) or k-rows (k-row image) past K clamped the same
// way, and those LDS slots are then overwritten with zeros.
#pragma once

#include "mfma_gemm.hpp"

namespace migemm {

#define MIGEMM_LDS __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// SCHED: 0 = a slab's LDS reads as one block, then its matrix instructions;
// 2 = one LDS read issued after each matrix instruction (sched_group_barrier);
// 4 = ping-pong: the two waves on each SIMD take turns, one issuing a whole
// k-tile of matrix instructions while the other reads its next k-tile of
// fragments (and, for the first group, issues the direct loads), with a
// barrier at each turn.
// FLAGS: bit 1 = non-temporal C stores; bit 2 = keep the accumulators in AGPRs
// (see below); bit 3 = issue a k-tile's direct loads right after the barrier
// that frees their stage instead of at the start of the next k-tile, so they
// have a whole k-tile of matrix work to land; bit 4 = also compiled for
// operands given transposed (without it those run the register-staged kernel);
// bit 5 = K need only be whole chunks: a last k-tile that K ends inside is
// zero-filled in LDS past K (interleaved schedules; compiled as a second
// instantiation of the kernel, launched only for such K); bit 6 = the same with
// the partial k-tile first instead (the k origin moved back so that the first
// k-tile holds the K mod BK leftover k and every later one is whole): its loads
// and zero fill happen in the prologue, so the k loop carries nothing for it;
// bit 7 = also compiled for split-K slices (GemmArgs::splitk).
template <typename E_, int BM_, int BN_, int WM_, int WN_, int MF_, int STAGES_ = 2,
          int BK_ = 64, int GM_ = 8, int SCHED_ = 0, int FLAGS_ = 0>
struct DirectCfg {
    using E = E_;
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MF = MF_, GM = GM_;
    static constexpr int STAGES = STAGES_, BK = BK_, SCHED = SCHED_, FLAGS = FLAGS_;
    static constexpr int NW = WM * WN, NT = NW * kWave;
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    static constexpr int TM = WTM / MF, TN = WTN / MF;
    static constexpr int EB = sizeof(E);  // bytes per element: 2 (FP16/BF16) or 1 (INT8)
    static constexpr int STAGE_A = BM * BK * EB, STAGE_B = BK * BN * EB;
    static constexpr int STAGE_BYTES = STAGE_A + STAGE_B;
    static constexpr bool LAYOUTS = (FLAGS & 16) != 0;
    // LDS placement.  Stage s of the other schedules is [A | B] at s * STAGE_BYTES.
    // Ping-pong keeps three B stages and two A stages: [B0 | B1 | B2 | A0 | A1].
    // B goes first so that a B fragment's slab and half offsets (up to 18 KiB)
    // stay within the 16-bit offset field of the LDS reads.
    static constexpr int LDS_BYTES = SCHED == 4 ? 2 * STAGE_A + 3 * STAGE_B : STAGES * STAGE_BYTES;
    __device__ static int a_stage(int kt) {
        return SCHED == 4 ? 3 * STAGE_B + (kt & 1) * STAGE_A : (kt % STAGES) * STAGE_BYTES;
    }
    __device__ static int b_stage(int kt) {
        return SCHED == 4 ? (kt % 3) * STAGE_B : (kt % STAGES) * STAGE_BYTES + STAGE_A;
    }
    static_assert(EB == 4 || EB == 2 || EB == 1, "32-, 16- or 8-bit inputs");
    static_assert(BM % (WM * MF) == 0 && BN % (WN * MF) == 0, "whole blocks per wave");
    static_assert(STAGES >= 2 && LDS_BYTES <= 160 * 1024, "stages fit 160 KiB");
    static_assert(SCHED == 0 || SCHED == 2 || SCHED == 4, "scheduling policy 0, 2 or 4");
    static_assert(SCHED != 4 || (WM == 2 && WN == 4 && STAGES == 2 && (FLAGS & 8) == 0),
                  "ping-pong: two groups of four waves, two stages, no early-load flag");
    static_assert((FLAGS & ~254) == 0, "flags: bits 1 to 7");
    static_assert(SCHED != 4 || (FLAGS & 96) == 0, "ping-pong: whole k-tiles");
    static_assert((FLAGS & 96) != 96, "a partial k-tile first or last, not both");
    static_assert((FLAGS & 128) == 0 || ((FLAGS & 16) != 0 && SCHED != 4),
                  "split-K slices: every layout, interleaved schedules");
};

// One operand's LDS image (BX rows of M or N by BK of k, EB-byte elements).
// KROW: [BX rows][BK EB / 16 chunks], k contiguous (row-major A, or B given
// transposed).  Otherwise a k-row image [BK k-rows][BX EB / 16 chunks], the BX
// side contiguous (row-major B, or A given transposed).  A direct load fills 64
// chunks: RPI image rows.  SWZ_PERIOD: the k-row swizzle repeats every so many
// k-rows.
template <int BX, int BK, int NW, bool KROW, int EB = 2>
struct DirectOperand {
    static constexpr bool ROWS = KROW;
    static constexpr int EPC = 16 / EB;                      // elements per 16-byte chunk
    static constexpr int CH = (KROW ? BK : BX) / EPC;        // 16-byte chunks per image row
    static constexpr int RPI = 64 / CH;
    static constexpr int INSTR = (KROW ? BX : BK) / RPI;
    static constexpr int PER = INSTR / NW;                   // direct loads per wave per k-tile
    static constexpr int SWZ_PERIOD = EB == 1 ? 32 : 16;
    static_assert(!KROW || CH == 4 || CH == 8, "row images are 64 or 128 bytes wide");
    static_assert(KROW || (EB == 2 ? (CH >= 8 && CH <= 64) : EB == 4 ? (CH >= 16 && CH <= 64)
                                                            : CH == 16),
                  "k-row images: 8 to 64 chunks (16-bit), 16 to 64 (32-bit), 16 (8-bit)");
    static_assert(INSTR % NW == 0, "loads split evenly over waves");
};

// Physical chunk of logical chunk c in row `row` of a row image (CA chunks per row).
// 128-byte rows (two rows per 256 bytes of banks): c ^ ((row >> 1) & 7).  64-byte
// rows (four rows per 256 bytes): c ^ ((row >> 2) & 3).  Either way sixteen
// consecutive rows reading one logical chunk cover the 64 banks once, and the
// pattern depends on row % 16 only.
template <int CA>
__device__ __forceinline__ int swz_a(int row) {
    if constexpr (CA == 8) return (row >> 1) & 7;
    return (row >> 2) & 3;
}
// Physical chunk of logical chunk c in k-row `krow` of a k-row image: c ^ swz_b(krow).
__device__ __forceinline__ int swz_b(int krow) { return ((krow & 3) | ((krow >> 1) & 4)) << 1; }
// For 16-bit k-row images 64 elements wide (128-byte k-rows, two per 256 bytes of
// banks): XOR the chunk pair with ((krow >> 1) & 1) | ((krow >> 3) & 1) << 1.  Of
// the 16 k-rows a transposing read takes (8 g + 4 h + 0..3 for the four groups
// g), each parity's eight rows then spread over the four chunk pairs of their
// half of the banks, two each: every bank twice, the minimum for 512 bytes.
__device__ __forceinline__ int swz_b64(int krow) { return (((krow >> 1) & 1) | (((krow >> 3) & 1) << 1)) << 1; }
// The same for 8-bit elements, 256-byte k-rows (16 chunks, one pass over the 64
// banks each).  A transposing 8-bit read takes one chunk from each of eight
// consecutive k-rows per lane group, rows 16g + 8h .. 16g + 8h + 7 for the four
// groups g: XOR with (krow & 7) | (bit 4 of krow) << 3 puts those 32 reads on 16
// distinct chunk positions, two each, the minimum for 512 bytes.
__device__ __forceinline__ int swz_b8(int krow) { return (krow & 7) | (((krow >> 4) & 1) << 3); }
// The same for 32-bit elements (k-rows of 16 or more chunks).  A fragment read
// takes, in lane group g, column j of k-row 16 s + 4 g + e (e = 0..3, one 4-byte
// read each): XOR with 4 ((krow >> 2) & 3) moves group g's four chunks to a
// quarter of the 64 banks of its own.
__device__ __forceinline__ int swz_b32(int krow) { return ((krow >> 2) & 3) << 2; }
// The k-row swizzle for operand O's element size.
template <class O>
__device__ __forceinline__ int swz_krow(int krow) {
    if constexpr (O::EPC == 8 && O::CH == 8) return swz_b64(krow);
    if constexpr (O::EPC == 8) return swz_b(krow);
    if constexpr (O::EPC == 4) return swz_b32(krow);
    return swz_b8(krow);
}

// Per-lane byte offsets of a wave's direct loads of one operand O, relative to
// its tile origin (row image: P + x0 * ld + k0; k-row image: P + k0 * ld + x0).
// Rows past the operand's extent `ext` (row image) and chunks past it (k-row
// image) are clamped, keeping every load in bounds.
template <class O>
__device__ __forceinline__ uint32_t direct_offset(int q, int wave, int lane, int nw, int64_t x0,
                                                  int64_t ext, int64_t ld) {
    constexpr int EPC = O::EPC, EB = 16 / EPC;
    const int r = O::RPI * (wave + q * nw) + lane / O::CH;
    if constexpr (O::ROWS) {
        const int chunk = (lane % O::CH) ^ swz_a<O::CH>(r);
        const int64_t gr = min(x0 + r, ext - 1);
        return static_cast<uint32_t>(((gr - x0) * ld + chunk * EPC) * EB);
    } else {
        const int chunk = (lane % O::CH) ^ swz_krow<O>(r);
        const int64_t gc = min(x0 + chunk * EPC, ext - EPC);
        return static_cast<uint32_t>((r * ld + (gc - x0)) * EB);
    }
}
template <class O>
__device__ __forceinline__ void direct_offsets(uint32_t (&voff)[O::PER], int wave, int lane, int nw,
                                               int64_t x0, int64_t ext, int64_t ld) {
#pragma unroll
    for (int q = 0; q < O::PER; ++q) voff[q] = direct_offset<O>(q, wave, lane, nw, x0, ext, ld);
}

// A last k-tile that K ends inside (K not a multiple of the k-tile, `tail` = K
// mod BK elements).  Whether the chunk that lane fetches in its q-th load
// starts below K: in a row image the lane's logical chunk of k (K is a whole
// number of chunks, or the operand a copy zero-filled past K to a whole chunk),
// in a k-row image its k-row.
template <class O>
__device__ __forceinline__ bool tail_valid(int q, int wave, int lane, int nw, int tail) {
    const int r = O::RPI * (wave + q * nw) + lane / O::CH;
    if constexpr (O::ROWS) return ((lane % O::CH) ^ swz_a<O::CH>(r)) * O::EPC < tail;
    return r < tail;
}
// The lane's offset (voff, from direct_offset) for that last k-tile: a chunk
// or k-row past K is replaced by the last one below K, so the load stays inside
// the operand; its LDS slot is zeroed once the load has landed.
template <class O>
__device__ __forceinline__ uint32_t tail_offset(uint32_t voff, int q, int wave, int lane, int nw,
                                                int tail, int64_t ld) {
    const int r = O::RPI * (wave + q * nw) + lane / O::CH;
    if constexpr (O::ROWS) {
        // the chunk holding k = K - 1 (zero-filled past K in a padded copy)
        const int chunk = (lane % O::CH) ^ swz_a<O::CH>(r), last = (tail - 1) / O::EPC;
        return chunk > last ? voff - static_cast<uint32_t>((chunk - last) * 16) : voff;
    } else {
        return r >= tail ? voff - static_cast<uint32_t>((r - (tail - 1)) * ld * (16 / O::EPC)) : voff;
    }
}

// A partial first k-tile (flag bit 6): the k origin sits `shift` = BK - K mod BK
// elements before k = 0, so the chunks (row image) or k-rows (k-row image) of
// the first k-tile that start below `shift` lie before the operand.  Whether
// the chunk that lane fetches in its q-th load is inside (K is a whole number of
// chunks, so a chunk is wholly before k = 0 or wholly after it).
template <class O>
__device__ __forceinline__ bool head_valid(int q, int wave, int lane, int nw, int shift) {
    const int r = O::RPI * (wave + q * nw) + lane / O::CH;
    if constexpr (O::ROWS) return ((lane % O::CH) ^ swz_a<O::CH>(r)) * O::EPC >= shift;
    return r >= shift;
}
// The lane's offset for the first k-tile: a chunk or k-row before k = 0 is
// replaced by the one at k = 0, so the load stays inside the operand; its LDS
// slot is zeroed once the load has landed.
template <class O>
__device__ __forceinline__ uint32_t head_offset(uint32_t voff, int q, int wave, int lane, int nw,
                                                int shift, int64_t ld) {
    const int r = O::RPI * (wave + q * nw) + lane / O::CH;
    if constexpr (O::ROWS) {
        const int chunk = (lane % O::CH) ^ swz_a<O::CH>(r), first = shift / O::EPC;
        return chunk < first ? voff + static_cast<uint32_t>((first - chunk) * 16) : voff;
    } else {
        return r < shift ? voff + static_cast<uint32_t>((shift - r) * ld * (16 / O::EPC)) : voff;
    }
}

// A wave-uniform address, moved to scalar registers (the direct loads take
// their base from an SGPR pair).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// 16 bytes per lane from global memory (SGPR base + per-lane byte offset) into
// LDS at lds_base + 16 * lane.  M0 carries the LDS base.  It is an input operand
// bound to M0 ("{m0}"), so the compiler itself writes M0 before the statement
// and knows what it holds afterwards: nothing the compiler keeps in M0 is
// overwritten behind its back.  The base is wave-uniform by construction;
// passing it through uniform_ptr keeps the compiler from handing the asm a VGPR
// copy of it, but the compiler often produces that SGPR pair with
// v_readfirstlane_b32 (a VALU instruction) right before the statement.
//
// Wait states.  The compiler inserts the waits its hazard rules require only
// around instructions it can see, not inside an asm statement, so the
// statement starts with its own: s_nop 4 is five wait states, what a vector
// memory instruction needs after a VALU instruction wrote an SGPR it reads (the
// address base here), and more than the one an LDS DMA needs after an SALU
// write of M0.  With fewer, the load can read a stale base and fault.
__device__ __forceinline__ void dma16(uint32_t lds_base, const void* sbase, uint32_t voff) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(uniform_ptr(sbase)), "{m0}"(lds_base)
                 : "memory");
}

// Wait until at most N of this wave's direct loads are outstanding (inline asm:
// the compiler does not track those loads), then until all its LDS reads have
// returned, then meet the other waves.  The LDS wait and the barrier use the
// builtins so the compiler's wait-count bookkeeping knows the reads completed;
// the empty asm statements keep memory operations from moving across.
__device__ __forceinline__ void lds_wait_then_barrier() {
    asm volatile("" : : : "memory");
    __builtin_amdgcn_s_waitcnt((0xF) | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" : : : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_then_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
    // s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maxima (gfx9 encoding)
    __builtin_amdgcn_s_waitcnt((0xF) | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" : : : "memory");
}

// TA: A given transposed (stored K x M); TB: B given transposed (stored N x K).
// KTAIL: K ends inside the last k-tile (configurations with flag bit 5 only; a
// separate instantiation, so products with whole k-tiles run code without it).
// KHEAD: the same with the partial k-tile first (flag bit 6).
// SPLITK: the grid is tiles x slices workgroups; workgroup w (renumbered
// XCD-contiguous, so that one XCD takes whole slices, whose tiles share rows of
// A and columns of B in its L2) takes tile w mod tiles of slice w / tiles of K
// (a whole number of 64 k, or of the k-tile where it is deeper; the last slice
// the rest, see splitk_slice) and writes its sums (FP32, INT32 for 8-bit
// inputs), plain, to that slice's M x N block of out.C (leading dimension N):
// the partial products that a reduction then sums.
template <class Cfg, bool GEN, bool TA, bool TB, bool KTAIL = false, bool KHEAD = false,
          bool SPLITK = false>
__global__ __launch_bounds__(Cfg::NT) void mfma16_direct_kernel(
    int64_t M, int64_t N, int64_t K, const typename Cfg::E* __restrict__ A, int64_t lda,
    const typename Cfg::E* __restrict__ B, int64_t ldb, Epi out, int tiles_m, int tiles_n) {
    int tile = blockIdx.x;
    if constexpr (SPLITK) {
        const int tiles = tiles_m * tiles_n;
        const int id = xcd_contiguous(blockIdx.x, gridDim.x), slice = id / tiles;
        tile = id - slice * tiles;
        const int64_t ks = splitk_slice(K, gridDim.x / tiles, Cfg::BK < 64 ? 64 : Cfg::BK);
        const int64_t k0 = slice * ks;
        A += TA ? k0 * lda : k0;
        B += TB ? k0 : k0 * ldb;
        K = K - k0 < ks ? K - k0 : ks;
        out.C = static_cast<float*>(out.C) + slice * M * N;
    }
    using E = typename Cfg::E;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, MF = Cfg::MF, TM = Cfg::TM, TN = Cfg::TN;
    constexpr int NW = Cfg::NW, S = Cfg::STAGES, BK = Cfg::BK;
    using OA = DirectOperand<BM, BK, NW, !TA, Cfg::EB>;
    using OB = DirectOperand<BN, BK, NW, TB, Cfg::EB>;
    constexpr int NI = OA::PER + OB::PER;  // direct loads per wave per k-tile
    static_assert((S - 2) * NI <= 63, "vmcnt counts at most 63 loads");
    using Op = MfmaOp<E, MF>;
    using Acc = typename Op::Acc;
    using L = AccLayout<MF>;

    __shared__ __attribute__((aligned(1024))) char smem[Cfg::LDS_BYTES];
    // __shared__ arrays are generic pointers in HIP; an LDS pointer needs a C-style cast.
    const MIGEMM_LDS char* const lds = (const MIGEMM_LDS char*)smem;
    const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm0 = (wave / Cfg::WN) * Cfg::WTM;
    const int wn0 = (wave % Cfg::WN) * Cfg::WTN;

    int pm, pn;
    if constexpr (SPLITK)
        band_coords<Cfg::GM>(tile, tiles_m, tiles_n, pm, pn);
    else
        tile_coords<Cfg::GM>(tile, tiles_m, tiles_n, pm, pn);
    const int64_t m0 = static_cast<int64_t>(pm) * BM;
    const int64_t n0 = static_cast<int64_t>(pn) * BN;

    // A k-row image's side is read in whole chunks: M or N rounded up (a no-op
    // unless the operand is a copy zero-filled to a whole chunk).
    constexpr int EPC = 16 / Cfg::EB;
    const int64_t ext_a = TA ? ceil_div(M, EPC) * EPC : M;
    const int64_t ext_b = TB ? N : ceil_div(N, EPC) * EPC;
    uint32_t a_voff[OA::PER], b_voff[OB::PER];
    direct_offsets<OA>(a_voff, wave, lane, NW, m0, ext_a, lda);
    direct_offsets<OB>(b_voff, wave, lane, NW, n0, ext_b, ldb);
    // KHEAD: the k origin moves back by `shift` elements, so that k-tile kt
    // covers k in [kt BK - shift, (kt + 1) BK - shift): the first k-tile holds
    // the K mod BK leftover k (the rest of its image is zeroed, see zero_head)
    // and every later one is whole, ending at K exactly.
    static_assert(!KHEAD || (!KTAIL && (Cfg::FLAGS & 64) != 0 && Cfg::SCHED != 4),
                  "a partial first k-tile only where flag bit 6 asks for it");
    const int shift = KHEAD ? static_cast<int>((BK - K % BK) % BK) : 0;
    // tile origins and the step from one k-tile to the next, in elements (with
    // KHEAD the origin is a k position before the operand; only offsets that
    // land inside it are ever added to it)
    const int64_t a_step = TA ? BK * lda : BK;
    const int64_t b_step = TB ? BK : BK * ldb;
    const E* const a_tile = (TA ? A + m0 : A + m0 * lda) - (KHEAD ? shift * a_step / BK : 0);
    const E* const b_tile = (TB ? B + n0 * ldb : B + n0) - (KHEAD ? shift * b_step / BK : 0);

    // KTAIL: K is not a multiple of the k-tile; the last k-tile holds `tail` of
    // its BK k, and the rest of its LDS image is zeroed (zero_tail) before it is
    // read, so those k add exact zero products.  Without it tail is 0 and none
    // of that code is compiled.
    static_assert(!KTAIL || ((Cfg::FLAGS & 32) != 0 && Cfg::SCHED != 4),
                  "a partial last k-tile only where flag bit 5 asks for it");
    const int KT = static_cast<int>(ceil_div(K, BK));
    const int tail = KTAIL ? static_cast<int>(K % BK) : 0;

    // For the last k-tile when K ends inside it: how far each of this wave's
    // per-lane load offsets moves back so that chunks or k-rows past K are
    // replaced by the last one below K (0 otherwise, and for whole k-tiles).
    // Held in registers and applied with a select, so the k loop has no branch
    // for it.
    uint32_t a_back[OA::PER], b_back[OB::PER];
#pragma unroll
    for (int q = 0; q < OA::PER; ++q)
        a_back[q] = tail ? a_voff[q] - tail_offset<OA>(a_voff[q], q, wave, lane, NW, tail, lda) : 0u;
#pragma unroll
    for (int q = 0; q < OB::PER; ++q)
        b_back[q] = tail ? b_voff[q] - tail_offset<OB>(b_voff[q], q, wave, lane, NW, tail, ldb) : 0u;

    // Issues this wave's NI direct loads of k-tile kt (A's, then B's) into its
    // stage; always NI loads, so the vmcnt accounting holds for the last k-tile too.
    auto issue = [&](int kt) __attribute__((always_inline)) {
        const int stage = kt % S;
        const uint32_t sa = lds_addr + stage * Cfg::STAGE_BYTES;
        const uint32_t sb = sa + Cfg::STAGE_A;
        const E* ab = a_tile + static_cast<int64_t>(kt) * a_step;
        const E* bb = b_tile + static_cast<int64_t>(kt) * b_step;
        const bool last = kt == KT - 1;
#pragma unroll
        for (int q = 0; q < OA::PER; ++q)
            dma16(sa + (wave + q * NW) * 1024, ab, a_voff[q] - (last ? a_back[q] : 0u));
#pragma unroll
        for (int q = 0; q < OB::PER; ++q)
            dma16(sb + (wave + q * NW) * 1024, bb, b_voff[q] - (last ? b_back[q] : 0u));
    };
    // Zeroes the LDS slots of the last k-tile that hold chunks or k-rows past K
    // (each lane its own slots: a direct load puts lane l's 16 bytes at the
    // load's LDS base + 16 l).  Called once that k-tile's loads have landed.
    auto zero_tail = [&]() __attribute__((always_inline)) {
        MIGEMM_LDS char* const st = (MIGEMM_LDS char*)smem + ((KT - 1) % S) * Cfg::STAGE_BYTES;
#pragma unroll
        for (int q = 0; q < OA::PER; ++q)
            if (!tail_valid<OA>(q, wave, lane, NW, tail))
                *(MIGEMM_LDS u32x4*)(st + (wave + q * NW) * 1024 + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < OB::PER; ++q)
            if (!tail_valid<OB>(q, wave, lane, NW, tail))
                *(MIGEMM_LDS u32x4*)(st + Cfg::STAGE_A + (wave + q * NW) * 1024 + 16 * lane) =
                    u32x4{0u, 0u, 0u, 0u};
    };
    // KHEAD: k-tile 0's loads into stage 0, a chunk or k-row before k = 0
    // replaced by the one at k = 0 (offsets computed here, in the prologue, and
    // not kept), and the zero fill of those slots once the loads have landed.
    auto issue_head = [&]() __attribute__((always_inline)) {
        const uint32_t sa = lds_addr, sb = sa + Cfg::STAGE_A;
#pragma unroll
        for (int q = 0; q < OA::PER; ++q)
            dma16(sa + (wave + q * NW) * 1024, a_tile,
                  head_offset<OA>(a_voff[q], q, wave, lane, NW, shift, lda));
#pragma unroll
        for (int q = 0; q < OB::PER; ++q)
            dma16(sb + (wave + q * NW) * 1024, b_tile,
                  head_offset<OB>(b_voff[q], q, wave, lane, NW, shift, ldb));
    };
    auto zero_head = [&]() __attribute__((always_inline)) {
        MIGEMM_LDS char* const st = (MIGEMM_LDS char*)smem;
#pragma unroll
        for (int q = 0; q < OA::PER; ++q)
            if (!head_valid<OA>(q, wave, lane, NW, shift))
                *(MIGEMM_LDS u32x4*)(st + (wave + q * NW) * 1024 + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < OB::PER; ++q)
            if (!head_valid<OB>(q, wave, lane, NW, shift))
                *(MIGEMM_LDS u32x4*)(st + Cfg::STAGE_A + (wave + q * NW) * 1024 + 16 * lane) =
                    u32x4{0u, 0u, 0u, 0u};
    };
    // The wait and barrier before the last k-tile is read, with at most P direct
    // loads left in flight.  Nothing is loaded after the last k-tile, so P is 0
    // whenever that k-tile is partial; then every load has landed and its slots
    // past K are zeroed before the barrier.
    auto land_last = [&](auto pending) __attribute__((always_inline)) {
        constexpr int P = decltype(pending)::value;
        if constexpr (P == 0) {
            if (tail != 0) {
                vm_wait<0>();
                zero_tail();
                lds_wait_then_barrier();
                return;
            }
        }
        wait_then_barrier<P>();
    };

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Acc{};
    if constexpr (Cfg::FLAGS & 4) {
        // The compiler gives matrix instructions AGPR accumulators only in
        // functions that may use AGPRs otherwise; an empty asm statement with an
        // AGPR operand makes this one such a function.  Accumulators in AGPRs keep
        // the C-operand traffic of the matrix instructions off the VGPR file that
        // the LDS reads write into.
        float agpr_hint = 0.0f;
        asm volatile("" : "+a"(agpr_hint));
    }

    // Fragment addressing.  MF = 16: lane (r + 16 g) feeds row r of a block (of A,
    // or column r of B) and the g-th 16-byte run of k of a slab: k = 8 g .. 8 g + 7
    // of a 32-k slab for 16-bit elements, k = 16 g .. 16 g + 15 of a 64-k slab for
    // 8-bit ones.  MF = 32 (16-bit only): lane (r + 32 g), k = 8 g .. of a 16-k
    // slab.  From a row image that is one 16-byte read; from a k-row image two
    // transposing reads, arranged so that lane j of each 16-lane group receives
    // column j of four (16-bit) or eight (8-bit) k-rows each time.
    constexpr int EB = Cfg::EB;
    static_assert(EB == 2 || MF == 16, "8-bit and 32-bit inputs use 16 x 16 instructions");
    constexpr int G = kWave / MF;          // k-groups per slab
    constexpr int SLAB_K = (16 / EB) * G;  // k per slab: 32 or 16 (16-bit), 64 (8-bit)
    constexpr int SLABS = BK / SLAB_K;
    const int ar = lane % MF, ag = lane / MF;
    const int bj = lane % 16;
    const int bcol = (MF == 16 ? 0 : 16 * ((lane % 32) / 16)) + 4 * (bj % 4);

    // Fragment `t` (block t of the wave tile starting at w0) of slab s from the
    // image `img` of a BX-wide operand.  Each address is written as the image
    // base, plus a per-lane part that stays the same for the whole loop, plus
    // a constant, so the compiler keeps a few per-lane offsets in registers and
    // folds the rest into instruction offsets:
    //  * row image: w0 + t MF is a multiple of 16 and the swizzle depends on
    //    row % 16 only, so the fragment's chunk is fixed by the lane and the
    //    slab, and t only adds t MF rows;
    //  * k-row image: the swizzle depends on k-row bits that come from the lane
    //    alone (bits 0, 1 and 3 of 8 ag + bj / 4 for 16-bit elements; bits 0-2
    //    and 4 of 16 ag + bj / 2 for 8-bit ones); the slab and half add whole
    //    k-rows; and with a power-of-two fragment count t sets column-chunk
    //    bits that nothing else sets, so it XORs the chunk index with the
    //    fragment's width in chunks times t.
    auto read_row_image = [&](const MIGEMM_LDS char* img, int w0, int t, int s)
        __attribute__((always_inline)) {
        constexpr int CA = BK * EB / 16;
        const int chunk = (s * G + ag) ^ swz_a<CA>(ar);
        const int lane_off = (w0 + ar) * (CA * 16) + chunk * 16;
        return *(const MIGEMM_LDS u32x4*)(img + lane_off + t * MF * (CA * 16));
    };
    auto read_krow_image = [&](const MIGEMM_LDS char* img, int bx, int w0, int t, int s)
        __attribute__((always_inline)) {
        u32x2 h[2];
        if constexpr (EB == 4) {
            // lane (j, g): column w0 + t MF + j of k-rows 16 s + 4 g + e, e = 0..3;
            // (k-row >> 2) & 3 = g, so the swizzle is the lane's own
            const int col = w0 + t * MF + bj;
            const int phys = (col >> 2) ^ (ag << 2);
            const int lane_off = (4 * ag) * (bx * 4) + phys * 16 + (col & 3) * 4;
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = *(const MIGEMM_LDS uint32_t*)(img + lane_off + (s * SLAB_K + e) * (bx * 4));
            return v;
        } else if constexpr (EB == 2) {
            // lane j of a group: column j of k-rows 4 half .. 4 half + 3 of its 8
            const int klane = 8 * ag + bj / 4;
            const int c0 = ((w0 + bcol) / 8) ^ (bx == 64 ? swz_b64(klane) : swz_b(klane));
            const int lane_off = klane * (bx * 2) + ((c0 ^ (t * MF / 8)) * 16) + (bcol % 8) * 2;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const MIGEMM_LDS char* p = img + lane_off + (s * SLAB_K + 4 * half) * (bx * 2);
                h[half] = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIGEMM_LDS s16x4*)p));
            }
        } else {
            // lane j of a group: column j of k-rows 8 half .. 8 half + 7 of its 16;
            // lanes 2e and 2e + 1 address the two 8-byte halves of k-row e's chunk
            const int klane = 16 * ag + bj / 2;
            const int c0 = (w0 / 16) ^ swz_b8(klane);
            const int lane_off = klane * bx + ((c0 ^ t) * 16) + 8 * (bj % 2);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const MIGEMM_LDS char* p = img + lane_off + (s * SLAB_K + 8 * half) * bx;
                h[half] = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((MIGEMM_LDS i32x2*)p));
            }
        }
        return u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
    };
    static_assert((TA ? (TM & (TM - 1)) : 0) == 0 && (TB ? 0 : (TN & (TN - 1))) == 0,
                  "k-row images need a power-of-two fragment count per wave");

    struct Frags {
        u32x4 a[TM];
        u32x4 b[TN];
    };
    auto load_frags = [&](int kt, int s, Frags& f) __attribute__((always_inline)) {
        // The stage offsets pass through an empty asm statement: otherwise loop
        // strength reduction turns every fragment address into an induction
        // variable of its own, and those registers spill.
        int a_off = Cfg::a_stage(kt), b_off = Cfg::b_stage(kt);
        asm("" : "+s"(a_off), "+s"(b_off));
        const MIGEMM_LDS char* sa = lds + a_off;
        const MIGEMM_LDS char* sb = lds + b_off;
        auto read_a = [&](int i) __attribute__((always_inline)) {
            f.a[i] = TA ? read_krow_image(sa, BM, wm0, i, s) : read_row_image(sa, wm0, i, s);
        };
        auto read_b = [&](int j) __attribute__((always_inline)) {
            f.b[j] = TB ? read_row_image(sb, wn0, j, s) : read_krow_image(sb, BN, wn0, j, s);
        };
        // Issued in the order the matrix instructions consume them (i-major):
        // a[0], then every b[j], then a[1] ...
        read_a(0);
#pragma unroll
        for (int j = 0; j < TN; ++j) read_b(j);
#pragma unroll
        for (int i = 1; i < TM; ++i) read_a(i);
    };
    auto mma = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) Op::run(acc[i][j], f.a[i], f.b[j]);
    };
    // One slab step: LDS reads of the next fragments (load) and this slab's
    // matrix instructions (f), ordered as the SCHED policy says.
    // LDS read instructions per slab: a row-image fragment is one 16-byte read,
    // a k-row-image one two transposing reads (16- and 8-bit) or four 4-byte
    // reads (32-bit); and matrix instructions per slab (four per fragment pair
    // for 32-bit elements)
    constexpr int kKrowReads = EB == 4 ? 4 : 2;
    constexpr int kReads = (TA ? kKrowReads : 1) * TM + (TB ? 1 : kKrowReads) * TN;
    constexpr int kMfma = TM * TN * (EB == 4 ? 4 : 1);
    auto slab_step = [&](bool do_load, int lkt, int ls, Frags& fl, const Frags& f) __attribute__((always_inline)) {
        if (do_load) load_frags(lkt, ls, fl);
        if constexpr (Cfg::SCHED == 2) {
            mma(f);
            // one matrix instruction, then one LDS read, while reads remain
#pragma unroll
            for (int r = 0; r < kReads; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if constexpr (kMfma > kReads)
                __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            __builtin_amdgcn_sched_barrier(0);
            mma(f);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Epilogue: the wave's accumulators to C (guarded at the matrix edges).
    // The general output step through LDS, for wave tiles 64 columns wide (see
    // store_tile).  Each wave uses 4 KiB of LDS of its own, 16 rows x 64 FP32
    // values, with the 16-byte chunk index XORed by (row >> 2) & 3 so that the
    // accumulator writes (lane group g: rows 4 g .. 4 g + 3) spread over four
    // bank quarters.  The LDS is free by then: in the ping-pong schedule every
    // wave's last fragment reads completed before the barrier that ended its
    // group's last reading turn; the other schedules meet a barrier first.
    // Per 16-row block i: the accumulators are written, then read back a row
    // piece per lane (8 outputs for 16-bit C, 4 for FP32 C: 16 bytes of C), with
    // the previous C of blocks i + 1 .. i + kAhead already loading.  The update
    // is store_update's arithmetic, so results are bit-identical to it.
    auto lds_epilogue = [&]() __attribute__((always_inline)) {
        if constexpr (Cfg::SCHED != 4) __syncthreads();
        constexpr bool NT = (Cfg::FLAGS & 2) != 0;
        constexpr int kAhead = TM >= 3 ? 2 : TM - 1, kRing = kAhead + 1;
        MIGEMM_LDS float* const scr =
            (MIGEMM_LDS float*)((MIGEMM_LDS char*)smem + wave * (16 * 64 * 4));
        const bool rd = out.beta != 0.0f;
        const int g = lane >> 4, jl = lane & 15;
        // HALF: 16-bit C, 2 passes of 8 rows x 8 columns per lane; otherwise FP32
        // C, 4 passes of 4 rows x 4 columns.  Pass p: this lane's row and first
        // column in the wave tile's 16 x 64 block.
        auto body = [&](auto half_tag) __attribute__((always_inline)) {
            constexpr bool HALF = decltype(half_tag)::value;
            constexpr int P = HALF ? 2 : 4, VE = HALF ? 8 : 4, ES = HALF ? 2 : 4;
            const int prow = HALF ? (lane >> 3) : (lane >> 4);
            const int c0 = HALF ? 8 * (lane & 7) : 4 * (lane & 15);
            const bool vec_c = (out.ldc * ES) % 16 == 0 &&
                               (reinterpret_cast<uintptr_t>(out.C) & 15) == 0;
            const int64_t gcol = n0 + wn0 + c0;
            const bool col_ok = vec_c && gcol + VE <= N;
            auto load_old = [&](int i, u32x4 (&o)[P]) __attribute__((always_inline)) {
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int64_t grow = m0 + wm0 + i * 16 + (16 / P) * p + prow;
                    o[p] = u32x4{0u, 0u, 0u, 0u};
                    if (rd && col_ok && grow < M)
                        o[p] = *reinterpret_cast<const u32x4*>(
                            static_cast<const char*>(out.C) + (grow * out.ldc + gcol) * ES);
                }
            };
            u32x4 ring[kRing][P];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) load_old(i, ring[i]);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if (i + kAhead < TM) load_old(i + kAhead, ring[(i + kAhead) % kRing]);
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        scr[(4 * g + r) * 64 + ((16 * j + jl) ^ (g << 4))] = acc[i][j][r];
                asm volatile("" : : : "memory");
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int row = (16 / P) * p + prow;
                    const int phys = c0 ^ (((row >> 2) & 3) << 4);
                    const int64_t grow = m0 + wm0 + i * 16 + row;
                    const int64_t idx = grow * out.ldc + gcol;
                    float v[VE];
                    {
                        const f32x4 v0 = *(const MIGEMM_LDS f32x4*)(scr + row * 64 + phys);
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = v0[e];
                        if constexpr (HALF) {
                            const f32x4 v1 = *(const MIGEMM_LDS f32x4*)(scr + row * 64 + phys + 4);
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[4 + e] = v1[e];
                        }
                    }
                    if (grow < M) {
                        if (col_ok) {
                            const u32x4 old = ring[i % kRing][p];
                            u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
                            for (int e = 0; e < VE; ++e) {
                                if constexpr (HALF) {
                                    const uint32_t ob = (old[e / 2] >> (16 * (e % 2))) & 0xffffu;
                                    const float prev =
                                        out.c_dtype == 1
                                            ? static_cast<float>(__builtin_bit_cast(
                                                  _Float16, static_cast<uint16_t>(ob)))
                                            : __uint_as_float(ob << 16);
                                    const float res = rd ? fmaf(out.alpha, v[e], out.beta * prev)
                                                         : out.alpha * v[e];
                                    const uint32_t nb =
                                        out.c_dtype == 1
                                            ? static_cast<uint32_t>(__builtin_bit_cast(
                                                  uint16_t, static_cast<_Float16>(res)))
                                            : static_cast<uint32_t>(f32_to_bf16_bits(res));
                                    w[e / 2] |= nb << (16 * (e % 2));
                                } else {
                                    const float res =
                                        rd ? fmaf(out.alpha, v[e], out.beta * __uint_as_float(old[e]))
                                           : out.alpha * v[e];
                                    w[e] = __float_as_uint(res);
                                }
                            }
                            u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(out.C) + idx * ES);
                            if constexpr (NT)
                                __builtin_nontemporal_store(w, dst);
                            else
                                *dst = w;
                        } else {
                            // edges and unaligned C, element by element (the values
                            // reread from LDS keep this loop rolled and small)
#pragma nounroll
                            for (int e = 0; e < VE; ++e)
                                if (gcol + e < N)
                                    store_update<NT>(out, idx + e, scr[row * 64 + (phys + e)],
                                                     rd ? load_prev(out, idx + e) : 0.0f);
                        }
                    }
                }
                asm volatile("" : : : "memory");
            }
        };
        if (out.c_dtype == 1 || out.c_dtype == 2)
            body(std::integral_constant<bool, true>{});
        else
            body(std::integral_constant<bool, false>{});
    };

    auto store_tile = [&]() __attribute__((always_inline)) {
        const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);
        const int lc = L::col(lane);
        constexpr bool NT = (Cfg::FLAGS & 2) != 0;
        auto inside = [&](int i, int j, int r) __attribute__((always_inline)) {
            return full_mn || (m0 + wm0 + i * MF + L::row(lane, r) < M && n0 + wn0 + j * MF + lc < N);
        };
        auto index = [&](int i, int j, int r) __attribute__((always_inline)) {
            return (m0 + wm0 + i * MF + L::row(lane, r)) * out.ldc + n0 + wn0 + j * MF + lc;
        };
        // The general step for wave tiles 64 columns wide (16x16 instructions,
        // 16- and 32-bit inputs): each 16-row block of the wave's accumulators
        // goes through LDS into row-major order, so the previous C is read and the
        // result written 16 bytes per lane in whole 128-byte lines, instead of 2- or
        // 4-byte accesses in 32- or 64-byte row pieces (the 16x16 accumulator
        // layout: four rows of one column per lane).
        constexpr bool kLdsEpilogue = GEN && MF == 16 && Cfg::WTN == 64 && EB != 1;
        if constexpr (kLdsEpilogue) {
            lds_epilogue();
        } else if constexpr (!GEN) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < L::R; ++r)
                        if (inside(i, j, r)) {
                        if constexpr (EB == 1) {  // exact INT32 sums of 8-bit products
                            int32_t* const p = static_cast<int32_t*>(out.C) + index(i, j, r);
                            if constexpr (NT)
                                store_i32_stream(p, acc[i][j][r]);
                            else
                                *p = acc[i][j][r];
                        } else
                            store_out<false, NT>(out, index(i, j, r), acc[i][j][r]);
                    }
        } else {
            // The general step reads the previous C (beta != 0) one row of fragments
            // at a time, keeping the loads of the next kAhead rows in flight while a
            // row is stored: the end-of-tile memory latency is paid about TM / kAhead
            // times per wave instead of once per element.  The fragment registers of
            // the main loop are free by now and hold the ring.
            constexpr int kAhead = TM >= 4 ? 3 : TM - 1;
            constexpr int kRing = kAhead + 1;
            const bool rd = out.beta != 0.0f;
            float prev[kRing][TN][L::R];
            auto load_row = [&](int i, float (&p)[TN][L::R]) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < L::R; ++r)
                        p[j][r] = (rd && inside(i, j, r)) ? load_prev(out, index(i, j, r)) : 0.0f;
            };
#pragma unroll
            for (int i = 0; i < kAhead; ++i) load_row(i, prev[i]);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if (i + kAhead < TM) load_row(i + kAhead, prev[(i + kAhead) % kRing]);
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < L::R; ++r)
                        if (inside(i, j, r))
                            store_update<NT>(out, index(i, j, r), acc[i][j][r],
                                             prev[i % kRing][j][r]);
            }
        }
    };

    if constexpr (Cfg::SCHED == 4) {
        // Ping-pong.  Waves 0-3 (group X, the upper BM/2 rows of the tile) and
        // waves 4-7 (group Y, the lower rows) share the four SIMDs pairwise.
        // Every wave holds a whole k-tile of fragments (both slabs).  Turns,
        // each ended by a barrier:
        //   turn 2 kt:     X runs k-tile kt's matrix instructions;
        //                  Y reads k-tile kt's fragments and issues B's direct
        //                  loads for k-tile kt + 2;
        //   turn 2 kt + 1: X reads k-tile kt + 1's fragments and issues A's
        //                  direct loads for k-tile kt + 2;
        //                  Y runs k-tile kt's matrix instructions.
        // So on each SIMD one wave issues nothing but matrix instructions while
        // the other reads LDS.  A direct load holds its wave's instruction issue
        // for about as long as a matrix instruction takes, so the loads ride in
        // the reading turns (one after every few fragment reads), which have
        // time to spare.  A has two LDS stages and B three: A's loads for
        // kt + 2 go to the stage of k-tile kt (last read by Y in turn 2 kt), B's
        // to the stage of k-tile kt - 1 (last read by Y in turn 2 kt - 2).  X
        // waits for its A loads at the end of turn 2 kt + 2, Y for its B loads
        // at the end of the same turn, before X reads k-tile kt + 2 in turn
        // 2 kt + 3.
        constexpr int NL = 4;  // waves per group
        using PA = DirectOperand<BM, BK, NL, !TA, Cfg::EB>;
        using PB = DirectOperand<BN, BK, NL, TB, Cfg::EB>;
        static_assert(PA::PER <= 16 && PB::PER <= 16, "direct loads per wave per k-tile");
        constexpr int PWA = PA::PER, PWB = PB::PER;  // direct loads per X / Y wave per k-tile
        static_assert(SLABS == 2, "a k-tile is two slabs of fragments");
        static_assert(Cfg::LDS_BYTES <= 160 * 1024, "two A and three B stages fit");
        const bool gx = wave < NL;
        // Whole tiles only (the launcher checks), so a wave's successive loads
        // of one operand are its first load moved by a fixed number of image
        // rows: that step goes into the scalar base, and only one per-lane
        // offset per swizzle pattern stays in a VGPR.  The row-image swizzle
        // repeats every 16 rows and a step is RPI * NL = 32 rows, so one
        // pattern; the k-row swizzle repeats every 16 (16-bit) or 32 (8-bit)
        // k-rows and a step is half that, so two (even and odd loads).
        static_assert(PA::ROWS ? (PA::RPI * NL) % 16 == 0 : (2 * PA::RPI * NL) % PA::SWZ_PERIOD == 0,
                      "swizzle patterns repeat with the load step");
        static_assert(PB::ROWS ? (PB::RPI * NL) % 16 == 0 : (2 * PB::RPI * NL) % PB::SWZ_PERIOD == 0,
                      "swizzle patterns repeat with the load step");
        const int wx = wave % NL;
        // X loads A, Y loads B: each wave keeps only its own operand's offsets.
        const uint32_t v0 = gx ? direct_offset<PA>(0, wx, lane, NL, m0, M, lda)
                               : direct_offset<PB>(0, wx, lane, NL, n0, N, ldb);
        const uint32_t v1 = gx ? direct_offset<PA>(1, wx, lane, NL, m0, M, lda)
                               : direct_offset<PB>(1, wx, lane, NL, n0, N, ldb);
        // Load q of this wave's share of operand O for k-tile kt: row image,
        // base moved q steps, pattern 0; k-row image, base moved 2 (q / 2)
        // steps, pattern q % 2.  A step is RPI * NL image rows, ld apart.
        auto dma_a = [&](int kt, int q) __attribute__((always_inline)) {
            const int64_t d = (PA::ROWS ? q : (q & ~1)) * int64_t(PA::RPI * NL) * lda;
            dma16(lds_addr + Cfg::a_stage(kt) + (wx + q * NL) * 1024,
                  a_tile + static_cast<int64_t>(kt) * a_step + d,
                  (PA::ROWS || (q & 1) == 0) ? v0 : v1);
        };
        auto dma_b = [&](int kt, int q) __attribute__((always_inline)) {
            const int64_t d = (PB::ROWS ? q : (q & ~1)) * int64_t(PB::RPI * NL) * ldb;
            dma16(lds_addr + Cfg::b_stage(kt) + (wx + q * NL) * 1024,
                  b_tile + static_cast<int64_t>(kt) * b_step + d,
                  (PB::ROWS || (q & 1) == 0) ? v0 : v1);
        };
        Frags P[2];
        // A k-tile of fragment reads; with `loads` 1 (A) or 2 (B) also the
        // wave's direct loads of k-tile kt_load (PWA of A or PWB of B), one after
        // every few
        // fragments.
        constexpr int kFrags = 2 * (TM + TN);
        auto read_ktile = [&](int kt, auto loads, int kt_load) __attribute__((always_inline)) {
            constexpr int L = decltype(loads)::value;
            constexpr int PW = L == 1 ? PWA : PWB;
            constexpr int EVERY = L ? (kFrags / PW > 0 ? kFrags / PW : 1) : 1;
            int r = 0, q = 0;
            auto after_read = [&]() __attribute__((always_inline)) {
                ++r;
                if (L && r % EVERY == 0 && q < PW) {
                    if constexpr (L == 1) dma_a(kt_load, q);
                    if constexpr (L == 2) dma_b(kt_load, q);
                    ++q;
                }
            };
            int a_off = Cfg::a_stage(kt), b_off = Cfg::b_stage(kt);
            asm("" : "+s"(a_off), "+s"(b_off));
            const MIGEMM_LDS char* sa = lds + a_off;
            const MIGEMM_LDS char* sb = lds + b_off;
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                Frags& f = P[sl];
                auto read_a = [&](int i) __attribute__((always_inline)) {
                    f.a[i] = TA ? read_krow_image(sa, BM, wm0, i, sl) : read_row_image(sa, wm0, i, sl);
                    after_read();
                };
                auto read_b = [&](int j) __attribute__((always_inline)) {
                    f.b[j] = TB ? read_row_image(sb, wn0, j, sl) : read_krow_image(sb, BN, wn0, j, sl);
                    after_read();
                };
                read_a(0);
#pragma unroll
                for (int j = 0; j < TN; ++j) read_b(j);
#pragma unroll
                for (int i = 1; i < TM; ++i) read_a(i);
            }
            // loads not yet issued (fewer fragments than loads x EVERY)
#pragma unroll
            for (int qq = 0; qq < PW; ++qq)
                if (qq >= q) {
                    if constexpr (L == 1) dma_a(kt_load, qq);
                    if constexpr (L == 2) dma_b(kt_load, qq);
                }
        };
        // A k-tile of matrix instructions.  With bar 1 (X: wait for its direct
        // loads, then the barrier) or 2 (Y: the barrier), the wave meets the
        // barrier that ends its turn kEarly instructions before its last one,
        // at raised priority: the other group then starts its turn while these
        // last instructions still fill the matrix pipe, and the raised priority
        // keeps them ahead of the other wave's first ones, so the barrier's
        // latency is hidden behind matrix work instead of leaving the pipe idle.
        constexpr int kEarly = 8;
        auto run_ktile = [&](auto bar) __attribute__((always_inline)) {
            constexpr int BK_ = decltype(bar)::value;
            __builtin_amdgcn_sched_barrier(0);
            int n = 0;
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        Op::run(acc[i][j], P[sl].a[i], P[sl].b[j]);
                        if (BK_ && n == 2 * TM * TN - 1 - kEarly) {
                            __builtin_amdgcn_sched_barrier(0);
                            __builtin_amdgcn_s_setprio(1);
                            if constexpr (BK_ == 1) wait_then_barrier<0>();
                            if constexpr (BK_ == 2) lds_wait_then_barrier();
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        ++n;
                    }
            __builtin_amdgcn_sched_barrier(0);
            if (BK_) __builtin_amdgcn_s_setprio(0);
        };
        using NoBarrier = std::integral_constant<int, 0>;
        using XBarrier = std::integral_constant<int, 1>;
        using YBarrier = std::integral_constant<int, 2>;
        using NoLoads = std::integral_constant<int, 0>;
        using ALoads = std::integral_constant<int, 1>;
        using BLoads = std::integral_constant<int, 2>;
        // Prologue: k-tiles 0 and 1 (X loads A, Y loads B); wait for k-tile 0.
        const int pro = KT > 1 ? 2 : 1;
        if (gx) {
            for (int t = 0; t < pro; ++t)
#pragma unroll
                for (int q = 0; q < PWA; ++q) dma_a(t, q);
        } else {
            for (int t = 0; t < pro; ++t)
#pragma unroll
                for (int q = 0; q < PWB; ++q) dma_b(t, q);
        }
        // each group waits for its own loads of k-tile 0
        if (KT > 1) {
            if (gx)
                vm_wait<PWA>();
            else
                vm_wait<PWB>();
        } else {
            vm_wait<0>();
        }
        lds_wait_then_barrier();
        // Each group runs its own straight-line loop (2 KT + 1 barriers in all
        // for both groups); the last two k-tiles, which load nothing, are
        // peeled so no branch splits a run of matrix instructions.
        if (gx) {
            read_ktile(0, NoLoads{}, -1);
            lds_wait_then_barrier();
            for (int kt = 0; kt + 2 < KT; ++kt) {
                run_ktile(XBarrier{});
                read_ktile(kt + 1, ALoads{}, kt + 2);
                lds_wait_then_barrier();
            }
            if (KT >= 2) {
                run_ktile(XBarrier{});
                read_ktile(KT - 1, NoLoads{}, -1);
                lds_wait_then_barrier();
            }
            run_ktile(XBarrier{});
            store_tile();
        } else {
            lds_wait_then_barrier();
            for (int kt = 0; kt + 2 < KT; ++kt) {
                read_ktile(kt, BLoads{}, kt + 2);
                // B of k-tile kt + 1 has landed; B of kt + 2 may still fly
                wait_then_barrier<PWB>();
                run_ktile(YBarrier{});
            }
            if (KT >= 2) {
                read_ktile(KT - 2, NoLoads{}, -1);
                wait_then_barrier<0>();
                run_ktile(YBarrier{});
            }
            read_ktile(KT - 1, NoLoads{}, -1);
            wait_then_barrier<0>();
            run_ktile(NoBarrier{});
            store_tile();
        }
        return;
    } else {
    // Prologue: k-tiles 0 .. S-2 in flight (0 .. S-1 with early loads, which
    // refill a stage right after the barrier that frees it); wait for k-tile 0.
    constexpr bool early = (Cfg::FLAGS & 8) != 0;
    constexpr int kPro = early ? S : S - 1;
    static_assert((kPro - 1) * NI <= 63, "vmcnt counts at most 63 loads");
#pragma unroll
    for (int t = 0; t < kPro; ++t)
        if (t < KT) {
            if (KHEAD && t == 0)
                issue_head();
            else
                issue(t);
        }
    if constexpr (KHEAD) {
        // k-tile 0 has landed (later ones may still fly); its slots before
        // k = 0 are zeroed before any wave reads it
        if (KT >= kPro)
            vm_wait<(kPro - 1) * NI>();
        else
            vm_wait<0>();
        zero_head();
        lds_wait_then_barrier();
    } else if (KT == 1) {
        land_last(std::integral_constant<int, 0>{});
    } else if (KT >= kPro) {
        wait_then_barrier<(kPro - 1) * NI>();
    } else {
        wait_then_barrier<0>();
    }

    // Two fragment buffers: slab s of every k-tile runs from F[s & 1] while the
    // next slab's fragments load into the other (SLABS is even, so slab 0 of
    // the next k-tile lands in F[0] again and no registers are copied).
    static_assert(SLABS % 2 == 0, "fragment ping-pong needs an even slab count");
    Frags F[2];
    load_frags(0, 0, F[0]);
    // All slabs of k-tile kt but the last, each reading the next slab's fragments.
    auto front_slabs = [&](int kt) {
#pragma unroll
        for (int s = 0; s + 1 < SLABS; ++s) slab_step(true, kt, s + 1, F[(s + 1) & 1], F[s & 1]);
    };
    // Every k-tile but the last ends with the barrier that makes k-tile kt+1
    // visible, then runs its last slab while slab 0 of kt+1 is read.  The last
    // k-tile is peeled off so that the code after the barrier has one
    // predecessor and the compiler's wait counts stay exact there.  With flag
    // bit 5 so is the step into it (LAST), whose wait also zero-fills a partial
    // last k-tile, so the loop itself has no branch for that.
    auto kstep = [&](int kt, auto last_tag) __attribute__((always_inline)) {
        constexpr bool LAST = decltype(last_tag)::value;
        const bool more = kt + S - 1 < KT;
        if (!early && more) issue(kt + S - 1);
        // sched_barrier(0) fences keep each slab's prefetch ahead of the
        // previous slab's matrix instructions instead of letting the scheduler
        // sink the LDS reads next to their first use.
        front_slabs(kt);
        // k-tile kt+1 must have landed; later ones (k-tiles up to kt+S-1) may
        // still be in flight.
        if constexpr (LAST) {
            if (more)
                land_last(std::integral_constant<int, (S - 2) * NI>{});
            else
                land_last(std::integral_constant<int, 0>{});
        } else {
            if (more)
                wait_then_barrier<(S - 2) * NI>();
            else
                wait_then_barrier<0>();
        }
        // Every read of k-tile kt's stage was issued before the barrier (the
        // last slab's fragments are already in registers) and has completed, in
        // every wave: the stage can take k-tile kt+S.
        if (early && kt + S < KT) issue(kt + S);
        slab_step(true, kt + 1, 0, F[0], F[1]);
    };
    if constexpr (KTAIL) {
        for (int kt = 0; kt + 2 < KT; ++kt) kstep(kt, std::false_type{});
        if (KT >= 2) kstep(KT - 2, std::true_type{});
    } else {
        // whole k-tiles: no step needs the zero fill, and one loop keeps the
        // code (and the registers live across it) as small as it can be
        for (int kt = 0; kt + 1 < KT; ++kt) kstep(kt, std::false_type{});
    }
    if (KT > 0) {
        front_slabs(KT - 1);
        slab_step(false, 0, 0, F[0], F[1]);
    }
    store_tile();
    }  // SCHED != 4

}

// True when the direct kernel's preconditions hold for these arguments: aligned
// operands with leading dimensions in whole 16-byte chunks (epc elements per
// chunk: 4 for 32-bit inputs, 8 for 16-bit ones, 16 for 8-bit ones), each
// operand's contiguous side (K for a row image, N for row-major B, M for A given
// transposed) in whole chunks unless the operand is a zero-filled copy (pad_a,
// pad_b), K a multiple of kq (the k-tile, for configurations without the
// partial last k-tile; kq = epc for those with it), and per-lane offsets
// (BX <= 256 rows of a row image, up to 128 k-rows of a k-row image) that fit
// 31 bits.  `layouts`: the configuration is compiled for operands given
// transposed.
inline bool direct_ok(const GemmArgs& g, int kq, bool layouts, int epc = 8) {
    if ((g.ta || g.tb) && !layouts) return false;
    const int64_t row_ld = int64_t(1) << 21, krow_ld = int64_t(1) << 23;
    // a padded copy's contiguous side may end inside a chunk (zero-filled)
    const bool a_whole = g.pad_a || (g.ta ? g.M : g.K) % epc == 0;
    const bool b_whole = g.pad_b || (g.tb ? g.K : g.N) % epc == 0;
    const bool k_ok = kq == epc || g.K % kq == 0;
    return aligned16(g.A) && aligned16(g.B) && g.lda % epc == 0 && g.ldb % epc == 0 &&
           k_ok && a_whole && b_whole && g.K > 0 && g.M > 0 && g.N > 0 &&
           (g.ta ? g.lda < krow_ld : g.lda < row_ld) && (g.tb ? g.ldb < row_ld : g.ldb < krow_ld);
}

// direct_ok for configuration D: K a whole number of chunks with flag bit 5 or
// 6, of k-tiles without (with bit 6 a whole number of chunks in every operand,
// zero-filled copies included: the first k-tile's split falls between chunks).
// The ping-pong schedule also needs whole tiles: its successive loads of a row
// image step whole image rows from the first one, with no clamp at the matrix
// edge.
template <class D>
bool direct_fits(const GemmArgs& g) {
    constexpr int kEpc = 16 / D::EB;
    const bool ragged = (D::FLAGS & 96) != 0;
    return direct_ok(g, ragged ? kEpc : D::BK, D::LAYOUTS, kEpc) &&
           (!(D::FLAGS & 64) || g.K % kEpc == 0) &&
           (D::SCHED != 4 || (g.M % D::BM == 0 && g.N % D::BN == 0));
}

template <class Cfg, bool GEN>
hipError_t launch_direct_cfg(const GemmArgs& g) {
    using E = typename Cfg::E;
    if (!direct_fits<Cfg>(g)) return hipErrorInvalidValue;
    const int64_t tm = ceil_div(g.M, Cfg::BM), tn = ceil_div(g.N, Cfg::BN);
    if (tm * tn > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(tm * tn)), block(Cfg::NT);
    const E* A = static_cast<const E*>(g.A);
    const E* B = static_cast<const E*>(g.B);
    const int itm = static_cast<int>(tm), itn = static_cast<int>(tn);
    // the partial-k-tile instantiation (last with flag bit 5, first with bit 6)
    // only where K ends inside a k-tile
    constexpr bool kTail = (Cfg::FLAGS & 32) != 0, kHead = (Cfg::FLAGS & 64) != 0;
    const bool ragged = (kTail || kHead) && g.K % Cfg::BK != 0;
    if constexpr ((Cfg::FLAGS & 128) != 0 && !GEN) {
        // split-K slices: tiles x slices workgroups; every slice but the last
        // is whole k-tiles, so the last decides the instantiation
        if (g.splitk > 1) {
            if (tm * tn * g.splitk > 0x7fffffff) return hipErrorInvalidValue;
            const dim3 sgrid(static_cast<unsigned>(tm * tn * g.splitk));
#define MIGEMM_SPLIT(TA_, TB_)                                                                 \
    return ragged ? launch_kernel(g, mfma16_direct_kernel<Cfg, false, TA_, TB_, kTail, kHead,  \
                                                          true>,                                \
                                  sgrid, block, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.out, itm, \
                                  itn)                                                         \
                  : launch_kernel(g, mfma16_direct_kernel<Cfg, false, TA_, TB_, false, false,  \
                                                          true>,                                \
                                  sgrid, block, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.out, itm, \
                                  itn)
            if (g.ta && g.tb)
                MIGEMM_SPLIT(true, true);
            else if (g.ta)
                MIGEMM_SPLIT(true, false);
            else if (g.tb)
                MIGEMM_SPLIT(false, true);
            else
                MIGEMM_SPLIT(false, false);
#undef MIGEMM_SPLIT
        }
    } else {
        if (g.splitk > 1) return hipErrorInvalidValue;  // not compiled for slices
    }
#define MIGEMM_LAUNCH(TA_, TB_)                                                                \
    return ragged ? launch_kernel(g, mfma16_direct_kernel<Cfg, GEN, TA_, TB_, kTail, kHead>,  \
                                  grid, block, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.out, itm, \
                                  itn)                                                        \
                  : launch_kernel(g, mfma16_direct_kernel<Cfg, GEN, TA_, TB_, false, false>,  \
                                  grid, block, g.M, g.N, g.K, A, g.lda, B, g.ldb, g.out, itm, \
                                  itn)
    if constexpr (Cfg::LAYOUTS) {
        if (g.ta && g.tb)
            MIGEMM_LAUNCH(true, true);
        else if (g.ta)
            MIGEMM_LAUNCH(true, false);
        else if (g.tb)
            MIGEMM_LAUNCH(false, true);
        else
            MIGEMM_LAUNCH(false, false);
    } else {
        if (g.ta || g.tb) return hipErrorInvalidValue;  // direct_ok sends these elsewhere
        MIGEMM_LAUNCH(false, false);
    }
#undef MIGEMM_LAUNCH
}

}  // namespace migemm
