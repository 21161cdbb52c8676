// mfma16.hip -- FP16/BF16 inputs, FP32 accumulation and output, on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_{f16,bf16} and
// v_mfma_f32_32x32x16_{f16,bf16}).
//
// Mixed precision as on page "CUDA-Practice 09" (section on why FP32
// accumulation is used): 16-bit inputs halve the bytes read, every product of
// two 16-bit values is exact in FP32, and the sums are kept in FP32 so long
// dot products do not lose small terms.  The pipeline is mfma_gemm.hpp:
// 128-byte (64-element) k-tiles, 16-byte coalesced global loads, B
// transposed in registers, swizzled double-buffered LDS, wave64 fragment
// mapping, XCD-aware tile order.
#include "mfma16_direct.hpp"

namespace migemm {
namespace {

template <typename E> struct Cfgs {
    using C0 = MfmaCfg<E, 256, 256, 2, 4, 16>;  // 8 waves, 128x64 per wave
    using C1 = MfmaCfg<E, 256, 256, 2, 2, 16>;  // 4 waves, 128x128 per wave
    using C2 = MfmaCfg<E, 256, 128, 2, 2, 16>;  // 4 waves, 128x64 per wave
    using C3 = MfmaCfg<E, 128, 128, 2, 2, 16>;  // 4 waves, 64x64 per wave
    using C4 = MfmaCfg<E, 64, 64, 2, 2, 16>;    // 4 waves, 32x32 per wave
    using C5 = MfmaCfg<E, 256, 256, 2, 4, 32>;  // 8 waves, 32x32x16 instructions
    using C6 = MfmaCfg<E, 128, 128, 2, 2, 32>;
    // direct global->LDS staging with transposing B reads (mfma16_direct.hpp)
    using D7 = DirectCfg<E, 256, 256, 2, 2, 16>;   // 4 waves, 128x128 per wave
    using D8 = DirectCfg<E, 256, 256, 2, 2, 32>;
    using D9 = DirectCfg<E, 256, 256, 2, 4, 16>;   // 8 waves, 128x64 per wave
    using D10 = DirectCfg<E, 256, 256, 2, 4, 32>;
    using D11 = DirectCfg<E, 128, 128, 2, 2, 16>;  // 4 waves, 64x64 per wave
    using D12 = DirectCfg<E, 256, 128, 2, 2, 16>;  // 4 waves, 128x64 per wave
    using D13 = DirectCfg<E, 128, 256, 2, 2, 16>;  // 4 waves, 64x128 per wave
};

template <typename E>
hipError_t launch_typed(const GemmArgs& g, int config) {
    using T = Cfgs<E>;
    switch (config) {
        case 1: return launch_mfma_cfg<typename T::C1>(g);
        case 2: return launch_mfma_cfg<typename T::C2>(g);
        case 3: return launch_mfma_cfg<typename T::C3>(g);
        case 4: return launch_mfma_cfg<typename T::C4>(g);
        case 5: return launch_mfma_cfg<typename T::C5>(g);
        case 6: return launch_mfma_cfg<typename T::C6>(g);
        default: break;
    }
    // Direct-staging configurations need aligned operands, K % 64 == 0 and
    // N % 8 == 0; otherwise the register-staged kernel with the same tile runs.
    const bool ok = direct_ok(g);
    switch (config) {
        case 7: return ok ? launch_direct_cfg<typename T::D7>(g) : launch_mfma_cfg<typename T::C0>(g);
        case 8: return ok ? launch_direct_cfg<typename T::D8>(g) : launch_mfma_cfg<typename T::C0>(g);
        case 9: return ok ? launch_direct_cfg<typename T::D9>(g) : launch_mfma_cfg<typename T::C0>(g);
        case 10: return ok ? launch_direct_cfg<typename T::D10>(g) : launch_mfma_cfg<typename T::C0>(g);
        case 11: return ok ? launch_direct_cfg<typename T::D11>(g) : launch_mfma_cfg<typename T::C3>(g);
        case 12: return ok ? launch_direct_cfg<typename T::D12>(g) : launch_mfma_cfg<typename T::C2>(g);
        case 13: return ok ? launch_direct_cfg<typename T::D13>(g) : launch_mfma_cfg<typename T::C3>(g);
        default: return launch_mfma_cfg<typename T::C0>(g);
    }
}

const char* const kNames[] = {"256x256x64 8w 16x16x32", "256x256x64 4w 16x16x32",
                              "256x128x64 4w 16x16x32", "128x128x64 4w 16x16x32",
                              "64x64x64 4w 16x16x32",   "256x256x64 8w 32x32x16",
                              "128x128x64 4w 32x32x16",
                              "direct 256x256x64 4w 16x16x32", "direct 256x256x64 4w 32x32x16",
                              "direct 256x256x64 8w 16x16x32", "direct 256x256x64 8w 32x32x16",
                              "direct 128x128x64 4w 16x16x32", "direct 256x128x64 4w 16x16x32",
                              "direct 128x256x64 4w 16x16x32"};

constexpr int kCount = sizeof(kNames) / sizeof(kNames[0]);

}  // namespace

int mfma16_config_count() { return kCount; }
const char* mfma16_config_name(int c) { return (c >= 0 && c < kCount) ? kNames[c] : nullptr; }

hipError_t launch_mfma16(const GemmArgs& g, int config) {
    return g.dtype == 1 ? launch_typed<_Float16>(g, config) : launch_typed<bf16_t>(g, config);
}

}  // namespace migemm
