// regtile_mfma.hip -- FP32 GEMM on the FP32 matrix-core instructions: the
// configuration names and the dispatch (each configuration's kernels are
// compiled in regtile_mfma_part.hip, one object per configuration and output
// form).  Configurations 0-7 stage tiles through registers; 8-11 load them
// straight into LDS (the direct-staged kernel of mfma16_direct.hpp on 32-bit
// elements) and need 16-byte aligned operands in whole 16-byte rows, K a
// multiple of 32 and the k-row image side (N for row-major B) a multiple of 4;
// other shapes run their register-staged fallback.
//
// The register-micro-tiled FP32 design (page "matmul_registers.cu",
// matmulRegTile2dVec4: 16-byte global loads, a k-major operand in LDS,
// per-lane register tiles of accumulators) with the inner product moved from
// VALU FMAs to v_mfma_f32_16x16x4_f32 / v_mfma_f32_32x32x2_f32.  On MI355X
// these run at 256 FLOP/clock/CU, twice the scalar-FMA VALU rate, and take
// their operands as one FP32 value per lane, so a 16-byte LDS read per lane
// feeds four instructions.  The staging pipeline is the one shared with the
// FP16/BF16 kernel (mfma_gemm.hpp): 128-byte k-tiles (BK = 32), swizzled
// double-buffered LDS, B transposed in registers on the way in.
#include "common.hpp"

namespace migemm {

template <bool GEN, int C>
hipError_t launch_f32_cfg(const GemmArgs& g);

namespace {

const char* const kNames[] = {"128x128x32 4w 16x16x4", "128x128x32 4w 32x32x2",
                              "64x64x32 4w 16x16x4", "256x128x32 4w 32x32x2",
                              "128x64x32 4w 16x16x4", "64x64x32 8w 16x16x4",
                              "128x128x32 8w 16x16x4", "64x32x32 4w 16x16x4",
                              "direct 64x64x32 8w 16x16x4 s4 ilv ntC",
                              "direct 64x64x32 4w 16x16x4 s4 ilv ntC",
                              "direct 128x128x32 8w 16x16x4 gm4 s4 ilv ntC",
                              "direct 128x64x32 8w 16x16x4 s4 ilv ntC",
                              "split-K: slices of K on config 8 into FP32 partials in the "
                              "workspace, then their sum",
                              "packed: aligned zero-padded copies, then config 10 or 8"};
constexpr int kCount = sizeof(kNames) / sizeof(kNames[0]);

template <bool GEN>
hipError_t launch_gen(const GemmArgs& g, int config) {
    switch (config) {
        case 1: return launch_f32_cfg<GEN, 1>(g);
        case 2: return launch_f32_cfg<GEN, 2>(g);
        case 3: return launch_f32_cfg<GEN, 3>(g);
        case 4: return launch_f32_cfg<GEN, 4>(g);
        case 5: return launch_f32_cfg<GEN, 5>(g);
        case 6: return launch_f32_cfg<GEN, 6>(g);
        case 7: return launch_f32_cfg<GEN, 7>(g);
        case 8: return launch_f32_cfg<GEN, 8>(g);
        case 9: return launch_f32_cfg<GEN, 9>(g);
        case 10: return launch_f32_cfg<GEN, 10>(g);
        case 11: return launch_f32_cfg<GEN, 11>(g);
        default: return launch_f32_cfg<GEN, 0>(g);
    }
}

}  // namespace

int regtile_mfma_config_count() { return kCount; }
const char* regtile_mfma_config_name(int c) { return (c >= 0 && c < kCount) ? kNames[c] : nullptr; }

namespace {

hipError_t launch_cfg(const GemmArgs& g, int config) {
    return g.general() ? launch_gen<true>(g, config) : launch_gen<false>(g, config);
}

}  // namespace

// The direct 128x128 (configuration 10) and 64x64 (8) tiles: a last band of tile
// rows or columns that would start a round of workgroups of its own is split
// off (split.cpp).  Tails of up to 16 run on the skinny kernel; wider ones on
// the 64x64 tile after the 128x128 one, and are left in place after the 64x64
// one (a tail on the same tile costs what the extra round does).
hipError_t launch_regtile_mfma(const GemmArgs& g, int config) {
    if (config == 13) return launch_packed32(g);
    if (config == 12) {
        // without a usable workspace the ordinary 64x64 launch
        const int64_t need = splitk32_workspace_bytes(g);
        if (need == 0 || g.ws == nullptr ||
            (reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign) != 0 || g.ws_bytes < need)
            return launch_regtile_mfma(g, 8);
        return launch_splitk32(g);
    }
    if (config == 8 || config == 10) {
        const int64_t t = config == 10 ? 128 : 64;
        const SplitPlan p = plan_split(g.M, g.N, t, t, config == 10 ? t : 16);
        if (p.rows || p.cols) return launch_split(g, p, launch_cfg, config, launch_cfg, 8);
    }
    return launch_cfg(g, config);
}

}  // namespace migemm
