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

hipError_t launch_mfma16(const GemmArgs& g, int config) {
    if (config == 11 || config == 12) {
        const int fallback = ceil_div(g.M, 128) * ceil_div(g.N, 128) >= 256 ? 2 : 3;
        return launch_packed16(g, config, fallback);
    }
    // Configuration 7 (128x128 tiles): a last band of tile rows that takes the
    // tile count just past a whole number of rounds of workgroups on the 256
    // CUs would run nearly alone in a round of its own (a 2050-row product: 16
    // of 272 tiles, about two thirds of a round's time).  Those rows go to a
    // launch of their own, after the whole 128-row bands, on the same stream:
    // up to 16 rows to the skinny kernel (K split over the waves of each
    // workgroup), more to the 64x64 tile (configuration 16).
    if (config == 7) {
        constexpr int64_t kCus = 256;
        const int64_t tn = ceil_div(g.N, 128), m_main = (g.M / 128) * 128;
        if (m_main > 0 && m_main < g.M &&
            ceil_div((m_main / 128) * tn, kCus) < ceil_div(ceil_div(g.M, 128) * tn, kCus)) {
            GemmArgs head = g, tail = g;
            head.M = m_main;
            tail.M = g.M - m_main;
            // row m_main of A: a column offset when A is given transposed (K x M)
            const int64_t a_off = g.ta ? m_main : m_main * g.lda;
            tail.A = static_cast<const char*>(g.A) + a_off * 2;  // FP16/BF16 elements
            const int64_t c_es = (g.out.c_dtype == 1 || g.out.c_dtype == 2) ? 2 : 4;
            tail.out.C = static_cast<char*>(g.out.C) + m_main * g.out.ldc * c_es;
            const hipError_t e = launch_mfma16(head, 7);
            if (e != hipSuccess) return e;
            return skinny16_fits(tail) ? launch_skinny16(tail) : launch_mfma16(tail, 16);
        }
    }
    return launch_cfg16_any(g, config);
}

}  // namespace migemm
