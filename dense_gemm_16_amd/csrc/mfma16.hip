// mfma16.hip -- FP16/BF16 inputs, FP32 accumulation, on the gfx950 matrix
// cores (v_mfma_f32_16x16x32_{f16,bf16} and v_mfma_f32_32x32x16_{f16,bf16}):
// the configuration names and the launcher, for the plain FP32 overwrite of C
// and for the general output step.
//
// Mixed precision as on page "CUDA-Practice 09" (section on why FP32
// accumulation is used): 16-bit inputs halve the bytes read, every product of
// two 16-bit values is exact in FP32, and the sums are kept in FP32 so long
// dot products do not lose small terms.
//
// Two pipelines:
// * register-staged (mfma_gemm.hpp): any shape, leading dimension and
//   alignment; 16-byte global loads into registers, B transposed in registers,
//   swizzled double-buffered LDS;
// * direct-staged (mfma16_direct.hpp): global->LDS without registers and
//   transposing LDS reads for B; needs 16-byte aligned operands, leading
//   dimensions in whole 16-byte chunks, K a multiple of 8 (configurations 7,
//   13 and 16, which zero-fill a partial last k-tile) or of the 64-deep k-tile
//   (the others), and N a multiple of 8.  A direct configuration asked to run
//   where these do not hold runs the register-staged kernel with the nearest
//   tile instead.
// Configurations 11 and 12 (pack.hip) first copy the operands the direct
// kernel cannot read in place (or reads slowly) into zero-padded k-contiguous
// images in a workspace the caller lends, so that the direct kernel applies to
// any layout, alignment and K.
//
// Every other configuration's kernels are compiled in mfma16_part.hip, one
// object per (element type, output form, configuration).
#include "mfma16_configs.hpp"

namespace migemm {
namespace {

const char* const kNames[] = {
    "256x256x64 8w 16x16x32",
    "256x128x64 4w 16x16x32",
    "128x128x64 4w 16x16x32",
    "64x64x64 4w 16x16x32",
    "256x256x64 8w 32x32x16",
    "direct 256x256x64 8w 16x16x32",
    "direct 256x256x64 8w 32x32x16",
    "direct 128x128x64 8w 16x16x32 gm4 s4 ilv ntC",
    "direct 128x128x64 4w 16x16x32 s4",
    "direct 256x256x64 8w 32x32x16 gm4 ilv ntC",
    "direct 256x256x64 8w 16x16x32 gm4 ilv ntC agpr early",
    "packed: zero-padded copies, then config 14 (whole tiles), 10 or 13 as A x B^T",
    "packed: zero-padded copies, then config 7 as A x B^T",
    "direct 128x256x64 8w 16x16x32 s3 ilv",
    "direct 256x256x64 8w 16x16x32 gm4 pingpong ntC agpr",
    "direct 128x256x64 8w 16x16x32 gm8 pingpong ntC agpr",
    "direct 64x64x64 8w 16x16x32 s4 early ntC"};
constexpr int kCount = sizeof(kNames) / sizeof(kNames[0]);

template <typename E, bool GEN>
hipError_t launch_typed(const GemmArgs& g, int config) {
    switch (config) {
#define MIGEMM_CASE(C) \
    case C: return launch_cfg16<E, GEN, C>(g);
        MIGEMM_CFG16_LIST(MIGEMM_CASE)
#undef MIGEMM_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int mfma16_config_count() { return kCount; }
const char* mfma16_config_name(int c) { return (c >= 0 && c < kCount) ? kNames[c] : nullptr; }

hipError_t launch_cfg16_any(const GemmArgs& g, int config) {
    if (g.general())
        return g.dtype == 1 ? launch_typed<_Float16, true>(g, config)
                            : launch_typed<bf16_t, true>(g, config);
    return g.dtype == 1 ? launch_typed<_Float16, false>(g, config)
                        : launch_typed<bf16_t, false>(g, config);
}

namespace {

constexpr int64_t kCus = 256;

// Tile of the direct configurations whose ragged last band is split off.
bool split_tile(int config, int64_t& bm, int64_t& bn) {
    switch (config) {
        case 7: bm = bn = 128; return true;
        case 10: case 14: bm = bn = 256; return true;
        case 13: case 15: bm = 128; bn = 256; return true;
        default: return false;
    }
}

int64_t element_bytes(int c_dtype) { return (c_dtype == 1 || c_dtype == 2) ? 2 : 4; }

// Rows [m0, M) of the product, every column.
hipError_t launch_row_tail(const GemmArgs& g, int64_t m0) {
    GemmArgs t = g;
    t.M = g.M - m0;
    // row m0 of A: a column offset when A is given transposed (K x M)
    t.A = static_cast<const char*>(g.A) + (g.ta ? m0 : m0 * g.lda) * 2;  // 16-bit elements
    t.out.C = static_cast<char*>(g.out.C) + m0 * g.out.ldc * element_bytes(g.out.c_dtype);
    return skinny16_fits(t) ? launch_skinny16(t) : launch_mfma16(t, 16);
}

// Columns [n0, N) of rows [0, m) of the product.  Up to 16 columns run as the
// transposed product C^T = B^T A^T on the skinny kernel: B's column slab is its
// left operand (k-contiguous rows when B is given transposed or is a packed
// copy, k-rows otherwise), A its right one, and C is written transposed.
hipError_t launch_col_tail(const GemmArgs& g, int64_t m, int64_t n0) {
    const char* const bslab = static_cast<const char*>(g.B) + (g.tb ? n0 * g.ldb : n0) * 2;
    char* const cslab = static_cast<char*>(g.out.C) + n0 * element_bytes(g.out.c_dtype);
    if (g.N - n0 <= 16) {
        GemmArgs t = g;
        t.M = g.N - n0;
        t.N = m;
        t.A = bslab;
        t.ta = !g.tb;
        t.lda = g.ldb;
        t.pad_a = g.pad_b;
        t.B = g.A;
        t.tb = !g.ta;
        t.ldb = g.lda;
        t.pad_b = g.pad_a;
        t.out.C = cslab;
        t.trans_c = true;
        if (skinny16_fits(t)) return launch_skinny16(t);
    }
    GemmArgs t = g;
    t.M = m;
    t.N = g.N - n0;
    t.B = bslab;
    t.out.C = cslab;
    return launch_mfma16(t, 16);
}

}  // namespace

hipError_t launch_mfma16(const GemmArgs& g, int config) {
    if (config == 11 || config == 12) {
        const int fallback = ceil_div(g.M, 128) * ceil_div(g.N, 128) >= 256 ? 2 : 3;
        return launch_packed16(g, config, fallback);
    }
    // A last band of tile rows (or columns) that takes the tile count just past
    // a whole number of rounds of workgroups on the 256 CUs would run nearly
    // alone in a round of its own: 4100 x 4096 on 256x256 tiles is 272 tiles,
    // and the 16 of the second round cost as much as the first 256.  The whole
    // tiles run first; the rows past them go to a launch of their own on the
    // same stream (up to 16 rows on the skinny kernel, which splits K over the
    // waves of each workgroup, more on the 64x64 tile, configuration 16), and
    // then the columns past them (up to 16 on the skinny kernel as the
    // transposed product, more on the 64x64 tile).  Whole 256x256 (128x256)
    // tiles and whole k-tiles run on the ping-pong kernel, configuration 14
    // (15), whichever of the two tile-shape configurations was asked for.
    int64_t bm, bn;
    if (split_tile(config, bm, bn)) {
        // whole and all tile rows (columns); split the rows, the columns or
        // both, whichever leaves the fewest rounds (fewer splits on a tie)
        const int64_t fm = g.M / bm, cm = ceil_div(g.M, bm), fn = g.N / bn, cn = ceil_div(g.N, bn);
        const bool can_m = fm > 0 && fm < cm, can_n = fn > 0 && fn < cn;
        int64_t best = ceil_div(cm * cn, kCus);
        bool split_m = false, split_n = false;
        auto consider = [&](bool m, bool n) {
            if ((m && !can_m) || (n && !can_n)) return;
            const int64_t r = ceil_div((m ? fm : cm) * (n ? fn : cn), kCus);
            if (r < best) {
                best = r;
                split_m = m;
                split_n = n;
            }
        };
        consider(true, false);
        consider(false, true);
        consider(true, true);
        const int64_t m_main = fm * bm, n_main = fn * bn;
        const int64_t mh = split_m ? m_main : g.M;
        if (split_m || split_n) {
            GemmArgs head = g;
            head.M = mh;
            head.N = split_n ? n_main : g.N;
            int hc = config;
            if (head.K % 64 == 0 && head.N % 256 == 0) {
                if (config == 10 && head.M % 256 == 0) hc = 14;
                if (config == 13 && head.M % 128 == 0) hc = 15;
            }
            hipError_t e = launch_cfg16_any(head, hc);
            if (e == hipSuccess && split_m) e = launch_row_tail(g, m_main);
            if (e == hipSuccess && split_n) e = launch_col_tail(g, mh, n_main);
            return e;
        }
    }
    return launch_cfg16_any(g, config);
}

}  // namespace migemm
