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
#include "mfma_gemm.hpp"

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
        default: return launch_mfma_cfg<typename T::C0>(g);
    }
}

const char* const kNames[] = {"256x256x64 8w 16x16x32", "256x256x64 4w 16x16x32",
                              "256x128x64 4w 16x16x32", "128x128x64 4w 16x16x32",
                              "64x64x64 4w 16x16x32",   "256x256x64 8w 32x32x16",
                              "128x128x64 4w 32x32x16"};

}  // namespace

int mfma16_config_count() { return 7; }
const char* mfma16_config_name(int c) { return (c >= 0 && c < 7) ? kNames[c] : nullptr; }

hipError_t launch_mfma16(const GemmArgs& g, int config) {
    return g.dtype == 1 ? launch_typed<_Float16>(g, config) : launch_typed<bf16_t>(g, config);
}

}  // namespace migemm
