// api.cpp -- the C ABI (migemm.h): argument checks, the variant registry,
// the deterministic selection table, stream-ordered launch, and the
// description of a call's kernels.
//
// The library's interface is a status-returning call in the manner of the
// vendor GEMM call on page "matmul_registers.cu" (section on the library
// comparison, where the status goes back to the caller rather than aborting):
// nothing here prints, throws or exits.  The library allocates no device
// memory: the one path that needs scratch memory (packed FP16/BF16 operands,
// pack.hip) takes it from a workspace the caller lends to migemm_gemm_ws, and
// runs a path that needs none when no workspace is lent.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "common.hpp"
#include "migemm.h"

namespace migemm {
namespace {

// Sizes are limited so that every index product fits in 64 bits:
// a dimension below 2^31 times a leading dimension below 2^32.
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxLd = int64_t(1) << 32;  // leading dimensions must be below this
// M * N * K from which a 16-bit product the direct kernel cannot read in place
// is run on packed copies (pack.hip) rather than by the register-staged kernel.
constexpr double kPackMinWork = 134217728.0;  // 2^27, e.g. 512^3
// M * N * K from which an INT8 product of fewer than 256 tiles of 256x256 runs
// on the direct 256x256 kernel (1792^3 = 5.75e9: 25.2 us against 31.0 for the
// 64x64 tile; 2048 x 1024 x 2048 = 4.3e9: 26.7 against 20.9).
constexpr double kI8DirectMinWork = 5.0e9;
// INT8 split-K: at most 64 tiles of 256x256 and K at least 8192.  Measured
// (us, split-K against the best other configuration): 512 x 512 x 8192 23.3
// against 68.3, 1024 x 1024 x 8192 38.7 against 68.6, 2048 x 2048 x 8192 54.3
// against 68.8, 256 x 256 x 65536 58.4 against 454; at K = 4096 and below it
// does not pay (1024 x 1024 x 4096 36.3 against 35.0, 2048 x 2048 x 4096 43.0
// against 41.0, 2048^3 37.9 against 26.8).
constexpr int64_t kSplitK8MaxTiles = 64, kSplitK8MinK = 8192;
// Shortest K for FP32 split-K.  An FP32 k-tile costs four times the matrix
// cycles of a 16-bit one, so the slices' sums cost little beside it: split-K
// measured faster on every product of at most 128 tiles of 64x64 tried from
// K = 512 (512^3: 9.9 against 11.5 us; 512 x 512 x 2048: 16.5 against 38.0;
// 1024 x 512 x 1024: 16.7 against 20.4; 512 x 512 x 65536: 288 against 1120).
constexpr int64_t kSplitKMinK32 = 512;
// Shortest K for split-K: below it the second launch and the slices' FP32 sums
// cost more than the longer walk of K by the 64x64 tile (BF16, 512 x 512 and
// 1024 x 1024: 16.6 against 20.8 and 19.4 us at K = 4096; 23.3 against 21.6 and
// 23.5 against 21.7 us at K = 6144).  Twice that where more than 128 tiles of
// 128x128 run as one partial round (1536 x 1536 x 8192: 56.6 us unsplit, 56.8
// split; 1536 x 1536 x 16384: 82.8 split).
constexpr int64_t kSplitKMinK = 6144;

struct Variant {
    const char* name;
    unsigned dtype_mask;  // bit d set: takes dtype d
    int (*count)();
    const char* (*config_name)(int);
    hipError_t (*launch)(const GemmArgs&, int);
};

const Variant kVariants[] = {
    {"naive", 0x7u, naive_config_count, naive_config_name, launch_naive},
    {"lds_tiled", 0x1u, lds_tiled_config_count, lds_tiled_config_name, launch_lds_tiled},
    {"regtile_valu", 0x1u, regtile_valu_config_count, regtile_valu_config_name,
     launch_regtile_valu},
    {"regtile_mfma", 0x1u, regtile_mfma_config_count, regtile_mfma_config_name,
     launch_regtile_mfma},
    {"mfma16", 0x6u, mfma16_config_count, mfma16_config_name, launch_mfma16},
    {"mfma_i8", 0x8u, mfma_i8_config_count, mfma_i8_config_name, launch_mfma_i8},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

thread_local int g_last_hip_error = 0;

int elem_size(int dtype) {
    return (dtype == MIGEMM_F32 || dtype == MIGEMM_I32) ? 4 : dtype == MIGEMM_I8 ? 1 : 2;
}

// INT8: each product is at most 2^14 in magnitude ((-128)(-128)), so sums of at
// most 2^17 - 1 of them stay below 2^31 and fit INT32 exactly.
constexpr int64_t kMaxKi8 = (int64_t(1) << 17) - 1;

// Byte range [lo, hi) touched by a rows x cols row-major operand (rows, cols >= 1)
// with leading dimension ld.  False when the range does not fit the address
// space: (rows - 1) ld + cols reaches 2^63 at the size limits, so the bytes are
// counted in 128 bits.
bool extent(const void* p, int64_t rows, int64_t cols, int64_t ld, int es, uintptr_t& lo,
            uintptr_t& hi) {
    lo = reinterpret_cast<uintptr_t>(p);
    const unsigned __int128 bytes =
        (static_cast<unsigned __int128>(rows - 1) * static_cast<unsigned __int128>(ld) +
         static_cast<unsigned __int128>(cols)) * static_cast<unsigned __int128>(es);
    if (bytes > static_cast<unsigned __int128>(UINTPTR_MAX - lo)) return false;
    hi = lo + static_cast<uintptr_t>(bytes);
    return true;
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

bool known_dtype(int d) { return d == MIGEMM_F32 || d == MIGEMM_F16 || d == MIGEMM_BF16; }
bool known_input(int d) { return known_dtype(d) || d == MIGEMM_I8; }
bool known_output(int d) { return known_dtype(d) || d == MIGEMM_I32; }

bool known_op(int op) { return op == MIGEMM_OP_N || op == MIGEMM_OP_T; }

// ta / tb: the operand is given transposed, so its stored rows run along k (A,
// stored K x M) or along n (B, stored N x K).
int check_args(int64_t M, int64_t N, int64_t K, int dtype, bool ta, bool tb, const void* A,
               int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc, int c_dtype,
               bool need_ptrs) {
    if (!known_input(dtype) || !known_output(c_dtype)) return MIGEMM_ERR_INVALID_ARG;
    // INT8 inputs go with INT32 C and nothing else does
    if ((dtype == MIGEMM_I8) != (c_dtype == MIGEMM_I32)) return MIGEMM_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return MIGEMM_ERR_INVALID_ARG;
    if (dtype == MIGEMM_I8 && K > kMaxKi8) return MIGEMM_ERR_INVALID_ARG;
    auto at_least = [](int64_t ld, int64_t cols) { return ld >= (cols > 1 ? cols : 1); };
    if (!at_least(lda, ta ? M : K) || !at_least(ldb, tb ? K : N) || !at_least(ldc, N))
        return MIGEMM_ERR_INVALID_ARG;
    if (lda >= kMaxLd || ldb >= kMaxLd || ldc >= kMaxLd) return MIGEMM_ERR_INVALID_ARG;
    if (!need_ptrs) return MIGEMM_OK;
    if ((M > 0 && K > 0 && !A) || (K > 0 && N > 0 && !B) || (M > 0 && N > 0 && !C))
        return MIGEMM_ERR_INVALID_ARG;
    if (M > 0 && N > 0) {
        const int es = elem_size(dtype);
        uintptr_t c0, c1;
        if (!extent(C, M, N, ldc, elem_size(c_dtype), c0, c1)) return MIGEMM_ERR_INVALID_ARG;
        if (K > 0) {
            uintptr_t a0, a1, b0, b1;
            const bool fit_a = ta ? extent(A, K, M, lda, es, a0, a1) : extent(A, M, K, lda, es, a0, a1);
            const bool fit_b = tb ? extent(B, N, K, ldb, es, b0, b1) : extent(B, K, N, ldb, es, b0, b1);
            if (!fit_a || !fit_b) return MIGEMM_ERR_INVALID_ARG;
            if (overlaps(c0, c1, a0, a1) || overlaps(c0, c1, b0, b1)) return MIGEMM_ERR_INVALID_ARG;
        }
    }
    return MIGEMM_OK;
}

// 16-byte aligned operand pointers with leading dimensions of whole 16-byte
// chunks (4 FP32, 8 16-bit or 16 8-bit elements).  NULL pointers count as
// aligned (migemm_select).
bool operands_aligned(const void* A, int64_t lda, const void* B, int64_t ldb, int dtype) {
    const int64_t epc = 16 / elem_size(dtype);
    return aligned16(A) && aligned16(B) && lda % epc == 0 && ldb % epc == 0;
}

}  // namespace

// INT8 configuration.  direct: the operands suit the direct kernels (16-byte
// aligned rows in whole chunks) and K is a multiple of the 128-deep k-tile;
// direct16: the same with K a multiple of 16 only.
//  * Whole 256x256 tiles: the direct ping-pong kernel (configuration 4).
//  * A ragged shape whose last bands are at most 16 rows or columns, or any
//    ragged shape of a round or more of 256x256 tiles: configuration 3, whose
//    launcher runs the whole tiles on the ping-pong kernel and the bands after
//    them (4100 x 4096 x 4096: 63.2 us, against 110.4 on configuration 6).
//  * Below a round of 256x256 tiles the direct kernels win once the product is
//    large or K long (one round takes about 12.7 us + 6.9 us per 1024 of K):
//    2048^3 26.9 us against 30.9 for the 64x64 tile, 3072^3 34.5 against 145
//    for the 128x128 one, 1024 x 1024 x 8192 68.7 against 138; and with wide
//    last bands the interleaved direct kernel (configuration 6: clamped loads,
//    guarded stores, a partial first k-tile) runs the whole shape in one
//    launch: 2000 x 2000 x 2048 39.3 us against 108 for the split, 3008 x 3008
//    x 3072 49.4 against 143.  It also takes K that is not a multiple of 128
//    (2048 x 2048 x 2000: 32.6 us against 38.8 on zero-padded copies).
//  * Smaller products: the register-staged 64x64 tile (1536^3 20.3 us against
//    26.8 on configuration 6), or 128x128 from a round of its tiles.
int i8_select(int64_t M, int64_t N, int64_t K, bool direct, bool direct16) {
    auto tiles = [&](int64_t bm, int64_t bn) { return ceil_div(M, bm) * ceil_div(N, bn); };
    const bool whole = M % 256 == 0 && N % 256 == 0;
    const bool narrow = M % 256 <= 16 && N % 256 <= 16;  // last bands for the skinny kernel
    const double work = static_cast<double>(M) * static_cast<double>(N) * static_cast<double>(K);
    const bool big = tiles(256, 256) >= 256;
    const bool large = M >= 256 && N >= 256 && (work >= kI8DirectMinWork || K >= 8192);
    if (direct && (big || large)) return whole ? 4 : (big || narrow) ? 3 : 6;
    if (direct16 && (big || large)) return 6;
    if (big) return 3;
    return tiles(128, 128) >= 256 ? 1 : 2;
}

namespace {

// The selection table: a pure function of shape, dtype, operand layout and
// alignment, and of whether the call lent a workspace large enough for the
// packed path.  Sizes are bucketed by how many workgroup tiles a configuration
// would launch against the 256 CUs of an MI355X.
void select(const GemmArgs& g, bool aligned, int& variant, int& config) {
    const int64_t M = g.M, N = g.N, K = g.K;
    const int dtype = g.dtype;
    const bool ta = g.ta, tb = g.tb;
    auto tiles = [&](int64_t bm, int64_t bn) { return ceil_div(M, bm) * ceil_div(N, bn); };
    if (dtype == MIGEMM_I8) {
        variant = MIGEMM_MFMA_I8;
        // Operands the direct kernels cannot read (K not a multiple of 16, rows
        // off 16-byte boundaries) are read a byte at a time by the
        // register-staged kernels (1000^3: 66.6 us against 11.4 for 1024^3);
        // once the product is large enough and a workspace is lent they are
        // copied into aligned zero-padded images first (configuration 5).
        const bool direct = K % 128 == 0 && aligned, direct16 = K % 16 == 0 && aligned;
        const double work = static_cast<double>(M) * static_cast<double>(N) * static_cast<double>(K);
        const bool pack = !direct16 && work >= kPackMinWork &&
                          ceil_div(K, 128) * 128 < (int64_t(1) << 21) && g.ws != nullptr &&
                          reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign == 0 &&
                          g.ws_bytes >= packed8_workspace_bytes(g);
        // split-K (configuration 7): few 256x256 tiles and a long K, where a
        // workspace for the slices' INT32 sums is lent
        const bool splitk = direct16 && tiles(256, 256) <= kSplitK8MaxTiles && K >= kSplitK8MinK &&
                            splitk8_workspace_bytes(g) > 0 && g.ws != nullptr &&
                            reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign == 0 &&
                            g.ws_bytes >= splitk8_workspace_bytes(g);
        config = pack ? 5 : splitk ? 7 : i8_select(M, N, K, direct, direct16);
        return;
    }
    if (dtype == MIGEMM_F32) {
        // Direct global->LDS staging (configurations 8-11) needs 16-byte aligned
        // operands in whole 16-byte rows, K a multiple of 4 (a last k-tile that K
        // ends inside is zero-filled in LDS) and the k-row image side (N for
        // row-major B, M for A given transposed) a multiple of 4; it measured 105
        // against 66 TFLOPS at 1024^3 (64x64 tiles, 8 waves) and 142 against 124
        // at 4096^3 (128x128 tiles).  Other operands stage through registers.
        variant = MIGEMM_REGTILE_MFMA;
        const bool direct = aligned && K % 4 == 0 && (tb || N % 4 == 0) && (!ta || M % 4 == 0);
        // split-K (configuration 12): at most half a round of 64x64 tiles, where a
        // workspace for the slices' sums is lent
        const bool splitk = direct && tiles(64, 64) <= 128 && K >= kSplitKMinK32 &&
                            splitk32_workspace_bytes(g) > 0 && g.ws != nullptr &&
                            reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign == 0 &&
                            g.ws_bytes >= splitk32_workspace_bytes(g);
        // operands it cannot read: copied first (configuration 13) once the
        // product is large enough and a workspace is lent
        const double work = static_cast<double>(M) * static_cast<double>(N) * static_cast<double>(K);
        const bool pack = !direct && work >= kPackMinWork &&
                          ceil_div(K, 32) * 32 < (int64_t(1) << 21) && g.ws != nullptr &&
                          reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign == 0 &&
                          g.ws_bytes >= packed32_workspace_bytes(g);
        if (direct)
            config = f32_direct_tile(M, N) == 10 ? 10 : splitk ? 12 : 8;
        else if (pack)
            config = 13;
        else
            config = tiles(128, 128) >= 256 ? 0 : 2;
        return;
    }
    variant = MIGEMM_MFMA16;
    // Direct global->LDS staging needs 16-byte aligned operands with leading
    // dimensions a multiple of 8 elements, K a multiple of 8 (of the 64-deep
    // k-tile for configurations 14 and 15; configurations 7, 13 and 16 zero-fill
    // a last k-tile that K ends inside, 10 a first one), and N (row-major B) or M
    // (A given transposed) a multiple of 8; the launcher falls back to the
    // register-staged kernel otherwise.  Other operands are packed into
    // zero-padded copies for the direct kernel once the product is large
    // enough for the extra copy launch to pay.
    const bool direct = aligned && K % 8 == 0 && (tb || N % 8 == 0) && (!ta || M % 8 == 0);
    const bool ktiles = K % 64 == 0;
    const double work = static_cast<double>(M) * static_cast<double>(N) * static_cast<double>(K);
    const int pc = tiles(256, 256) >= 256 ? 11 : 12;  // packed copies, then config 14/10 or 7
    // (copies' leading dimensions: K, M or N rounded up to 64, within the direct
    // kernel's offset limits)
    const bool pack = work >= kPackMinWork && packed_k(K) < (int64_t(1) << 21) &&
                      packed_k(M > N ? M : N) < (int64_t(1) << 23) &&
                      packed16_workspace_ok(g, pc);
    const bool whole256 = M % 256 == 0 && N % 256 == 0;
    // split-K (splitk.hip): a k-sum long beside a product of few 128x128 tiles,
    // where a workspace for the slices' FP32 sums is lent (twice as long where
    // the 128x128 tile alone already fills more than half a round)
    const bool splitk = direct && tiles(128, 128) < 256 &&
                        K >= (tiles(128, 128) > 128 ? 2 * kSplitKMinK : kSplitKMinK) &&
                        K >= 4 * (M > N ? M : N) && splitk16_workspace_bytes(g) > 0 &&
                        g.ws != nullptr &&
                        reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign == 0 &&
                        g.ws_bytes >= splitk16_workspace_bytes(g);
    // Whole tiles below one round of 256x256 but at least one of 128x128: the
    // tile whose rounds of workgroups (one per CU) cost least, from each tile's
    // time per full round per unit of K (ns: 256x256 ping-pong 21.4 at 8192^3,
    // 128x256 ping-pong 13.4 at 1024x8192x8192, 128x128 9.7 at 2048^3)
    int small_whole = 0;
    if (direct && ktiles && tiles(256, 256) < 256 && tiles(128, 128) >= 256 &&
        M % 128 == 0 && N % 256 == 0) {
        auto cost = [&](int64_t bm, int64_t bn, double ns) {
            return static_cast<double>(ceil_div(tiles(bm, bn), 256)) * ns;
        };
        const double c7 = cost(128, 128, 9.7), c15 = cost(128, 256, 13.4);
        const double c14 = whole256 ? cost(256, 256, 21.4) : 1e300;
        small_whole = c14 <= c15 && c14 <= c7 ? 14 : c15 <= c7 ? 15 : 7;
    }
    if (small_whole)
        config = small_whole;
    else if (direct && ktiles && tiles(256, 256) >= 256 && whole256)
        config = 14;  // direct 256x256x64, ping-pong wave groups (whole tiles only)
    else if (direct && tiles(256, 256) >= 256)
        config = 10;  // direct 256x256x64, 8 waves, 16x16x32, AGPR accumulators, early loads
                      // (a K that ends inside a k-tile: the partial k-tile first)
    else if (direct && ktiles && tiles(128, 256) >= 256 && M % 128 == 0 && N % 256 == 0)
        config = 15;  // direct 128x256x64, ping-pong wave groups (e.g. 1024x8192, 4096x2048)
    else if (direct && tiles(128, 256) >= 256)
        config = 13;  // direct 128x256x64, 8 waves of 64x64, 3 stages
    else if (direct && tiles(128, 128) >= 256)
        config = 7;   // direct 128x128x64, 8 waves, 4 stages, interleaved
    else if (splitk)
        config = 17;  // slices of K on the direct 128x128 or 256x256 tile, then their sum
    else if (direct && tiles(128, 128) > 128)
        config = 7;   // one partial round of 128x128 tiles rather than 3 or 4 of 64x64
    else if (direct)
        config = 16;  // direct 64x64x64, 8 waves: four times the workgroups (e.g. 1024^3)
    else if (pack)
        config = pc;
    else if (tiles(128, 128) >= 256)
        config = 2;   // register-staged 128x128x64
    else
        config = 3;   // register-staged 64x64x64
}

// Validates one call and resolves its variant and configuration into g.
// need_ptrs: check pointers and overlap (a launch); false for the queries,
// where NULL pointers stand for 256-byte aligned ones.
int prepare(int& variant, int& config, int op_a, int op_b, int64_t M, int64_t N, int64_t K,
            int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, float alpha,
            float beta, int c_dtype, void* C, int64_t ldc, void* ws, int64_t ws_bytes,
            void* stream, bool need_ptrs, GemmArgs& g) {
    if (!known_op(op_a) || !known_op(op_b)) return MIGEMM_ERR_INVALID_ARG;
    const bool ta = op_a == MIGEMM_OP_T, tb = op_b == MIGEMM_OP_T;
    int st = check_args(M, N, K, dtype, ta, tb, A, lda, B, ldb, C, ldc, c_dtype, need_ptrs);
    if (st != MIGEMM_OK) return st;
    if (ws_bytes < 0) return MIGEMM_ERR_INVALID_ARG;
    // INT32 C takes the plain product only
    if (c_dtype == MIGEMM_I32 && (alpha != 1.0f || beta != 0.0f)) return MIGEMM_ERR_UNSUPPORTED;
    if (!need_ptrs) {
        // stand-ins with the alignment a fresh allocation has (pointer arithmetic only)
        if (!A) A = reinterpret_cast<const void*>(uintptr_t(1) << 40);
        if (!B) B = reinterpret_cast<const void*>(uintptr_t(2) << 40);
        if (!C) C = reinterpret_cast<void*>(uintptr_t(3) << 40);
        if (!ws && ws_bytes > 0) ws = reinterpret_cast<void*>(uintptr_t(4) << 40);
    }
    g = GemmArgs{M,   N,   K, dtype, ta, tb, A, lda, B, ldb,
                 Epi{C, ldc, alpha, beta, c_dtype}, static_cast<hipStream_t>(stream)};
    g.ws = ws;
    g.ws_bytes = ws ? ws_bytes : 0;
    const bool aligned = operands_aligned(A, lda, B, ldb, dtype);
    if (variant == MIGEMM_VARIANT_AUTO) {
        if (config != -1) return MIGEMM_ERR_INVALID_ARG;
        select(g, aligned, variant, config);
    }
    if (variant < 0 || variant >= kNumVariants) return MIGEMM_ERR_INVALID_ARG;
    const Variant& v = kVariants[variant];
    if (!(v.dtype_mask & (1u << dtype))) return MIGEMM_ERR_UNSUPPORTED;
    if (config == -1) {
        int sv, sc;
        select(g, aligned, sv, sc);
        config = (sv == variant) ? sc : 0;
    }
    if (config < 0 || config >= v.count()) return MIGEMM_ERR_INVALID_ARG;
    return MIGEMM_OK;
}

// Launches the product g with the variant's configuration (or, for K == 0, the
// empty product; nothing for an empty C).
hipError_t launch(const GemmArgs& g, int variant, int config) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    return g.K == 0 ? launch_empty_product(g) : kVariants[variant].launch(g, config);
}

// Workspace bytes the call's configuration uses when lent at least that many:
// the packed FP16/BF16 configurations' copies, nothing for the others.
int64_t config_workspace_bytes(const GemmArgs& g, int variant, int config) {
    if (g.M == 0 || g.N == 0 || g.K == 0) return 0;
    if (variant == MIGEMM_REGTILE_MFMA && config == 12) return splitk32_workspace_bytes(g);
    if (variant == MIGEMM_REGTILE_MFMA && config == 13) return packed32_workspace_bytes(g);
    if (variant == MIGEMM_MFMA_I8 && config == 5) return packed8_workspace_bytes(g);
    if (variant == MIGEMM_MFMA_I8 && config == 7) return splitk8_workspace_bytes(g);
    if (variant != MIGEMM_MFMA16 || (config != 11 && config != 12 && config != 17)) return 0;
    if (config == 17) return splitk16_workspace_bytes(g);
    return packed16_workspace_bytes(g, config);
}

// key=value pairs, separated by ';', describing the call's kernels.
std::string describe(const GemmArgs& g0, int variant, int config) {
    GemmArgs g = g0;
    LaunchInfo info;
    g.query = &info;
    (void)launch(g, variant, config);
    char tmp[256];
    std::string out;
    auto put = [&](const char* key, const std::string& value) {
        if (!out.empty()) out += ';';
        out += key;
        out += '=';
        out += value;
    };
    auto num = [&](long long v) {
        snprintf(tmp, sizeof tmp, "%lld", v);
        return std::string(tmp);
    };
    put("variant", kVariants[variant].name);
    put("config", num(config));
    put("config_name", kVariants[variant].config_name(config));
    put("workspace_bytes", num(config_workspace_bytes(g0, variant, config)));
    put("workspace_lent", num(g0.ws ? g0.ws_bytes : 0));
    put("launches", num(info.count));
    for (int i = 0; i < info.count && i < LaunchInfo::kMax; ++i) {
        const std::string k = num(i);
        put(("grid" + k).c_str(), num(info.grid[i]));
        put(("block" + k).c_str(), num(info.block[i]));
        hipFuncAttributes attr{};
        hipError_t e = hipFuncGetAttributes(&attr, info.fn[i]);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            put(("resources" + k).c_str(), "unavailable (hipError_t " + num(e) + ")");
            continue;
        }
        const char* name = hipKernelNameRefByPtr(info.fn[i], nullptr);
        (void)hipGetLastError();
        if (name) put(("kernel" + k).c_str(), name);
        put(("regs" + k).c_str(), num(attr.numRegs));
        put(("lds_bytes" + k).c_str(), num(static_cast<long long>(attr.sharedSizeBytes)));
        put(("scratch_bytes" + k).c_str(), num(static_cast<long long>(attr.localSizeBytes)));
        put(("max_block" + k).c_str(), num(attr.maxThreadsPerBlock));
        int blocks = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, info.fn[i],
                                                         static_cast<int>(info.block[i]), 0) ==
            hipSuccess) {
            put(("workgroups_per_cu" + k).c_str(), num(blocks));
            put(("waves_per_simd" + k).c_str(),
                num(static_cast<long long>(blocks) * ((info.block[i] + kWave - 1) / kWave) / 4));
        } else {
            (void)hipGetLastError();
        }
    }
    return out;
}

int write_text(const std::string& text, char* buf, int buflen) {
    if (!buf || buflen <= 0) return MIGEMM_ERR_INVALID_ARG;
    const size_t n = text.size() < static_cast<size_t>(buflen - 1) ? text.size()
                                                                    : static_cast<size_t>(buflen - 1);
    text.copy(buf, n);
    buf[n] = '\0';
    return n == text.size() ? MIGEMM_OK : MIGEMM_ERR_INVALID_ARG;
}

}  // namespace

int run_gemm(int variant, int config, int op_a, int op_b, int64_t M, int64_t N, int64_t K,
             int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, float alpha,
             float beta, int c_dtype, void* C, int64_t ldc, void* ws, int64_t ws_bytes,
             void* stream) {
    GemmArgs g{};
    const int st = prepare(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha,
                           beta, c_dtype, C, ldc, ws, ws_bytes, stream, true, g);
    if (st != MIGEMM_OK) return st;
    const hipError_t err = launch(g, variant, config);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return MIGEMM_ERR_HIP;
    }
    return MIGEMM_OK;
}

int workspace_bytes(int variant, int config, int op_a, int op_b, int64_t M, int64_t N,
                    int64_t K, int dtype, const void* A, int64_t lda, const void* B,
                    int64_t ldb, int64_t* bytes) {
    if (!bytes) return MIGEMM_ERR_INVALID_ARG;
    GemmArgs g{};
    // as if an unbounded workspace were lent, so the selection may pick the packed path
    const int c_dtype = dtype == MIGEMM_I8 ? MIGEMM_I32 : MIGEMM_F32;
    const int st = prepare(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, 1.0f,
                           0.0f, c_dtype, nullptr, N > 1 ? N : 1, nullptr, INT64_MAX, nullptr,
                           false, g);
    if (st != MIGEMM_OK) return st;
    *bytes = config_workspace_bytes(g, variant, config);
    return MIGEMM_OK;
}

}  // namespace migemm

using namespace migemm;

extern "C" {

int migemm_gemm(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                const void* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
    return run_gemm(MIGEMM_VARIANT_AUTO, -1, MIGEMM_OP_N, MIGEMM_OP_N, M, N, K, dtype, A, lda, B,
                    ldb, 1.0f, 0.0f, MIGEMM_F32, C, ldc, nullptr, 0, stream);
}

int migemm_gemm_variant(int variant, int config, int64_t M, int64_t N, int64_t K, int dtype,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                        int64_t ldc, void* stream) {
    return run_gemm(variant, config, MIGEMM_OP_N, MIGEMM_OP_N, M, N, K, dtype, A, lda, B, ldb,
                    1.0f, 0.0f, MIGEMM_F32, C, ldc, nullptr, 0, stream);
}

int migemm_gemm_ex(int op_a, int op_b, int64_t M, int64_t N, int64_t K, int dtype, const void* A,
                   int64_t lda, const void* B, int64_t ldb, float alpha, float beta, int c_dtype,
                   void* C, int64_t ldc, void* stream) {
    return run_gemm(MIGEMM_VARIANT_AUTO, -1, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha,
                    beta, c_dtype, C, ldc, nullptr, 0, stream);
}

int migemm_gemm_ex_variant(int variant, int config, int op_a, int op_b, int64_t M, int64_t N,
                           int64_t K, int dtype, const void* A, int64_t lda, const void* B,
                           int64_t ldb, float alpha, float beta, int c_dtype, void* C,
                           int64_t ldc, void* stream) {
    return run_gemm(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha, beta,
                    c_dtype, C, ldc, nullptr, 0, stream);
}

int migemm_gemm_ws(int variant, int config, int op_a, int op_b, int64_t M, int64_t N, int64_t K,
                   int dtype, const void* A, int64_t lda, const void* B, int64_t ldb,
                   float alpha, float beta, int c_dtype, void* C, int64_t ldc, void* workspace,
                   int64_t workspace_bytes, void* stream) {
    return run_gemm(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha, beta,
                    c_dtype, C, ldc, workspace, workspace_bytes, stream);
}

int migemm_workspace_size(int variant, int config, int op_a, int op_b, int64_t M, int64_t N,
                          int64_t K, int dtype, const void* A, int64_t lda, const void* B,
                          int64_t ldb, int64_t* bytes) {
    return workspace_bytes(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, bytes);
}

int migemm_describe(int64_t M, int64_t N, int64_t K, int dtype, int64_t lda, int64_t ldb,
                    int64_t ldc, char* buf, int buflen) {
    const int c_dtype = dtype == MIGEMM_I8 ? MIGEMM_I32 : MIGEMM_F32;
    return migemm_describe_ex(MIGEMM_VARIANT_AUTO, -1, MIGEMM_OP_N, MIGEMM_OP_N, M, N, K, dtype,
                              nullptr, lda, nullptr, ldb, c_dtype, ldc, 0, buf, buflen);
}

int migemm_describe_ex(int variant, int config, int op_a, int op_b, int64_t M, int64_t N,
                       int64_t K, int dtype, const void* A, int64_t lda, const void* B,
                       int64_t ldb, int c_dtype, int64_t ldc, int64_t workspace_bytes, char* buf,
                       int buflen) {
    if (!buf || buflen <= 0) return MIGEMM_ERR_INVALID_ARG;
    buf[0] = '\0';
    GemmArgs g{};
    const float alpha = 1.0f, beta = 0.0f;
    const int st = prepare(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha,
                           beta, c_dtype, nullptr, ldc, nullptr, workspace_bytes, nullptr, false,
                           g);
    if (st != MIGEMM_OK) return st;
    return write_text(describe(g, variant, config), buf, buflen);
}

int migemm_convert(int src_dtype, int dst_dtype, int64_t rows, int64_t cols, const void* src,
                   int64_t lds, void* dst, int64_t ldd, void* stream) {
    if (!known_dtype(src_dtype) || !known_dtype(dst_dtype)) return MIGEMM_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return MIGEMM_ERR_INVALID_ARG;
    const int64_t min_ld = cols > 1 ? cols : 1;
    if (lds < min_ld || ldd < min_ld || lds >= kMaxLd || ldd >= kMaxLd) return MIGEMM_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return MIGEMM_OK;
    if (!src || !dst) return MIGEMM_ERR_INVALID_ARG;
    uintptr_t s0, s1, d0, d1;
    extent(src, rows, cols, lds, elem_size(src_dtype), s0, s1);
    extent(dst, rows, cols, ldd, elem_size(dst_dtype), d0, d1);
    if (overlaps(s0, s1, d0, d1)) return MIGEMM_ERR_INVALID_ARG;
    const hipError_t err = launch_convert(src_dtype, dst_dtype, rows, cols, src, lds, dst, ldd,
                                          static_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return MIGEMM_ERR_HIP;
    }
    return MIGEMM_OK;
}

int migemm_variant_count(void) { return kNumVariants; }

const char* migemm_variant_name(int variant) {
    return (variant >= 0 && variant < kNumVariants) ? kVariants[variant].name : nullptr;
}

int migemm_variant_supports(int variant, int dtype) {
    if (variant < 0 || variant >= kNumVariants || !known_input(dtype)) return 0;
    return (kVariants[variant].dtype_mask >> dtype) & 1u;
}

int migemm_config_count(int variant) {
    return (variant >= 0 && variant < kNumVariants) ? kVariants[variant].count() : 0;
}

const char* migemm_config_name(int variant, int config) {
    if (variant < 0 || variant >= kNumVariants) return nullptr;
    return kVariants[variant].config_name(config);
}

int migemm_select(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                  const void* B, int64_t ldb, const float* C, int64_t ldc, int* variant,
                  int* config) {
    if (!variant || !config) return MIGEMM_ERR_INVALID_ARG;
    const int c_dtype = dtype == MIGEMM_I8 ? MIGEMM_I32 : MIGEMM_F32;
    int v = MIGEMM_VARIANT_AUTO, c = -1;
    GemmArgs g{};
    const int st = prepare(v, c, MIGEMM_OP_N, MIGEMM_OP_N, M, N, K, dtype, A, lda, B, ldb, 1.0f,
                           0.0f, c_dtype, const_cast<float*>(C), ldc, nullptr, 0, nullptr, false,
                           g);
    if (st != MIGEMM_OK) return st;
    *variant = v;
    *config = c;
    return MIGEMM_OK;
}

const char* migemm_status_string(int status) {
    switch (status) {
        case MIGEMM_OK: return "ok";
        case MIGEMM_ERR_INVALID_ARG: return "invalid argument";
        case MIGEMM_ERR_UNSUPPORTED: return "variant does not support this dtype";
        case MIGEMM_ERR_HIP: return "HIP runtime error";
        case MIGEMM_ERR_WORKSPACE:
            return "the product needs more scratch memory than the allocation-free entry point holds";
        default: return "unknown status";
    }
}

int migemm_last_hip_error(void) { return g_last_hip_error; }

int migemm_version(void) { return 600; }

}  // extern "C"
