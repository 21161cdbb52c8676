// regtile_mfma.hip -- FP32 GEMM on the FP32 matrix-core instructions.
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
#include "mfma_gemm.hpp"

namespace migemm {
namespace {

using F0 = MfmaCfg<float, 128, 128, 2, 2, 16>;  // 4 waves, 64x64 per wave
using F1 = MfmaCfg<float, 128, 128, 2, 2, 32>;
using F2 = MfmaCfg<float, 64, 64, 2, 2, 16>;    // small problems: 4x the workgroups
using F3 = MfmaCfg<float, 256, 128, 2, 2, 32>;  // 128x64 per wave
using F4 = MfmaCfg<float, 128, 64, 2, 2, 16>;
using F5 = MfmaCfg<float, 64, 64, 2, 4, 16>;    // 8 waves of 32x16: two waves per SIMD
using F6 = MfmaCfg<float, 128, 128, 2, 4, 16>;  // 8 waves of 64x32
using F7 = MfmaCfg<float, 64, 32, 2, 2, 16>;    // 4 waves of 32x16, twice F2's workgroups

const char* const kNames[] = {"128x128x32 4w 16x16x4", "128x128x32 4w 32x32x2",
                              "64x64x32 4w 16x16x4", "256x128x32 4w 32x32x2",
                              "128x64x32 4w 16x16x4", "64x64x32 8w 16x16x4",
                              "128x128x32 8w 16x16x4", "64x32x32 4w 16x16x4"};
constexpr int kCount = sizeof(kNames) / sizeof(kNames[0]);

template <bool GEN>
hipError_t launch_gen(const GemmArgs& g, int config) {
    switch (config) {
        case 1: return launch_mfma_cfg<F1, GEN>(g);
        case 2: return launch_mfma_cfg<F2, GEN>(g);
        case 3: return launch_mfma_cfg<F3, GEN>(g);
        case 4: return launch_mfma_cfg<F4, GEN>(g);
        case 5: return launch_mfma_cfg<F5, GEN>(g);
        case 6: return launch_mfma_cfg<F6, GEN>(g);
        case 7: return launch_mfma_cfg<F7, GEN>(g);
        default: return launch_mfma_cfg<F0, GEN>(g);
    }
}

}  // namespace

int regtile_mfma_config_count() { return kCount; }
const char* regtile_mfma_config_name(int c) { return (c >= 0 && c < kCount) ? kNames[c] : nullptr; }

hipError_t launch_regtile_mfma(const GemmArgs& g, int config) {
    return g.general() ? launch_gen<true>(g, config) : launch_gen<false>(g, config);
}

}  // namespace migemm
