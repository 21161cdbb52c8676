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
    "direct 64x64x64 8w 16x16x32 s4 early ntC",
    "split-K: slices of K on config 7 or 10 into FP32 partials in the workspace, then their sum"};
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

// Tile of the direct configurations whose ragged last band is split off.
bool split_tile(int config, int64_t& bm, int64_t& bn) {
    switch (config) {
        case 7: bm = bn = 128; return true;
        case 10: case 14: bm = bn = 256; return true;
        case 13: case 15: bm = 128; bn = 256; return true;
        default: return false;
    }
}

}  // namespace

hipError_t launch_mfma16(const GemmArgs& g, int config) {
    if (config == 17) {
        // without a usable workspace the ordinary 128x128 launch
        const int64_t need = splitk16_workspace_bytes(g);
        if (need == 0 || g.ws == nullptr ||
            (reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign) != 0 || g.ws_bytes < need)
            return launch_mfma16(g, 7);
        return launch_splitk16(g);
    }
    if (config == 11 || config == 12) {
        const int fallback = ceil_div(g.M, 128) * ceil_div(g.N, 128) >= 256 ? 2 : 3;
        return launch_packed16(g, config, fallback);
    }
    // The 128x128, 128x256 and 256x256 tiles: a last band of tile rows or
    // columns that would start a round of workgroups of its own is split off
    // (split.cpp), tails wider than 16 running on the 64x64 tile (configuration
    // 16).  Whole 256x256 (128x256) tiles with whole k-tiles run on the
    // ping-pong kernel, configuration 14 (15), whichever of the two tile-shape
    // configurations was asked for.
    int64_t bm, bn;
    if (split_tile(config, bm, bn)) {
        const SplitPlan p = plan_split(g.M, g.N, bm, bn, int64_t(1) << 62);
        if (p.rows || p.cols) {
            int hc = config;
            if (g.K % 64 == 0 && p.n_main % 256 == 0) {
                if (config == 10 && p.m_main % 256 == 0) hc = 14;
                if (config == 13 && p.m_main % 128 == 0) hc = 15;
            }
            return launch_split(g, p, launch_cfg16_any, hc, launch_cfg16_any, 16);
        }
    }
    return launch_cfg16_any(g, config);
}

}  // namespace migemm
