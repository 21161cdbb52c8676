// mfma16.hip -- FP16/BF16 inputs, FP32 accumulation and output, on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_{f16,bf16} and
// v_mfma_f32_32x32x16_{f16,bf16}).
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
//   dimensions in whole 16-byte chunks, K a multiple of the k-tile and N a
//   multiple of 8.  A direct configuration asked to run where these do not hold
//   runs the register-staged kernel with the nearest tile instead.
#include "mfma16_direct.hpp"

namespace migemm {
namespace {

template <typename E> struct Cfgs {
    // register-staged
    using C0 = MfmaCfg<E, 256, 256, 2, 4, 16>;  // 8 waves, 128x64 per wave
    using C1 = MfmaCfg<E, 256, 256, 2, 2, 16>;  // 4 waves, 128x128 per wave
    using C2 = MfmaCfg<E, 256, 128, 2, 2, 16>;  // 4 waves, 128x64 per wave
    using C3 = MfmaCfg<E, 128, 128, 2, 2, 16>;  // 4 waves, 64x64 per wave
    using C4 = MfmaCfg<E, 64, 64, 2, 2, 16>;    // 4 waves, 32x32 per wave
    using C5 = MfmaCfg<E, 256, 256, 2, 4, 32>;  // 8 waves, 32x32x16 instructions
    using C6 = MfmaCfg<E, 128, 128, 2, 2, 32>;
    // direct-staged: <E, BM, BN, WM, WN, MF, STAGES, BK>
    using D7 = DirectCfg<E, 256, 256, 2, 2, 16, 2, 64>;
    using D8 = DirectCfg<E, 256, 256, 2, 2, 32, 2, 64>;
    using D9 = DirectCfg<E, 256, 256, 2, 4, 16, 2, 64>;
    using D10 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64>;
    using D11 = DirectCfg<E, 128, 128, 2, 2, 16, 2, 64>;
    using D12 = DirectCfg<E, 256, 128, 2, 2, 16, 2, 64>;
    using D13 = DirectCfg<E, 128, 256, 2, 2, 16, 2, 64>;
    using D14 = DirectCfg<E, 256, 256, 2, 4, 32, 4, 32>;  // 8 waves, 4 stages of 32 k
    using D15 = DirectCfg<E, 256, 256, 2, 4, 32, 5, 32>;  // 8 waves, 5 stages of 32 k
    using D16 = DirectCfg<E, 256, 256, 2, 2, 32, 4, 32>;  // 4 waves, 4 stages of 32 k
    using D17 = DirectCfg<E, 256, 256, 2, 2, 32, 5, 32>;  // 4 waves, 5 stages of 32 k
    using D18 = DirectCfg<E, 128, 128, 2, 2, 16, 3, 64>;  // 3 stages
    using D19 = DirectCfg<E, 128, 128, 2, 2, 16, 4, 64>;  // 4 stages
    using D20 = DirectCfg<E, 256, 128, 2, 2, 32, 3, 64>;  // 3 stages, 128x64 per wave
    // scheduling and tile-order variants of D10
    using D21 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64, 8, 1>;   // s_setprio
    using D22 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64, 8, 2>;   // interleave
    using D23 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64, 8, 3>;   // interleave + prio
    using D24 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64, 4, 0>;   // 4-row bands
    using D25 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64, 16, 0>;  // 16-row bands
    using D26 = DirectCfg<E, 256, 256, 2, 2, 32, 2, 64, 8, 3>;   // 4 waves, interleave + prio
    using D27 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64, 4, 2, 1>;  // spread direct loads
    using D28 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64, 4, 2, 2>;  // non-temporal C
    using D29 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64, 4, 2, 3>;  // both
    using D30 = DirectCfg<E, 256, 256, 2, 4, 32, 4, 32, 4, 2, 2>;  // BK 32 x 4 stages, nt C
    using D31 = DirectCfg<E, 256, 256, 2, 2, 32, 2, 64, 4, 3, 3>;  // 4 waves, all of it
    // 16x16x32 instructions with AGPR accumulators and early direct loads
    using D32 = DirectCfg<E, 256, 256, 2, 4, 16, 2, 64, 4, 2, 14>;
};

template <class D, class Fallback>
hipError_t direct_or(const GemmArgs& g) {
    return direct_ok(g, D::BK) ? launch_direct_cfg<D>(g) : launch_mfma_cfg<Fallback>(g);
}

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
        case 7: return direct_or<typename T::D7, typename T::C0>(g);
        case 8: return direct_or<typename T::D8, typename T::C0>(g);
        case 9: return direct_or<typename T::D9, typename T::C0>(g);
        case 10: return direct_or<typename T::D10, typename T::C0>(g);
        case 11: return direct_or<typename T::D11, typename T::C3>(g);
        case 12: return direct_or<typename T::D12, typename T::C2>(g);
        case 13: return direct_or<typename T::D13, typename T::C3>(g);
        case 14: return direct_or<typename T::D14, typename T::C0>(g);
        case 15: return direct_or<typename T::D15, typename T::C0>(g);
        case 16: return direct_or<typename T::D16, typename T::C0>(g);
        case 17: return direct_or<typename T::D17, typename T::C0>(g);
        case 18: return direct_or<typename T::D18, typename T::C3>(g);
        case 19: return direct_or<typename T::D19, typename T::C3>(g);
        case 20: return direct_or<typename T::D20, typename T::C2>(g);
        case 21: return direct_or<typename T::D21, typename T::C0>(g);
        case 22: return direct_or<typename T::D22, typename T::C0>(g);
        case 23: return direct_or<typename T::D23, typename T::C0>(g);
        case 24: return direct_or<typename T::D24, typename T::C0>(g);
        case 25: return direct_or<typename T::D25, typename T::C0>(g);
        case 26: return direct_or<typename T::D26, typename T::C0>(g);
        case 27: return direct_or<typename T::D27, typename T::C0>(g);
        case 28: return direct_or<typename T::D28, typename T::C0>(g);
        case 29: return direct_or<typename T::D29, typename T::C0>(g);
        case 30: return direct_or<typename T::D30, typename T::C0>(g);
        case 31: return direct_or<typename T::D31, typename T::C0>(g);
        case 32: return direct_or<typename T::D32, typename T::C0>(g);
        default: return launch_mfma_cfg<typename T::C0>(g);
    }
}

const char* const kNames[] = {
    "256x256x64 8w 16x16x32",          "256x256x64 4w 16x16x32",
    "256x128x64 4w 16x16x32",          "128x128x64 4w 16x16x32",
    "64x64x64 4w 16x16x32",            "256x256x64 8w 32x32x16",
    "128x128x64 4w 32x32x16",          "direct 256x256x64 4w 16x16x32",
    "direct 256x256x64 4w 32x32x16",   "direct 256x256x64 8w 16x16x32",
    "direct 256x256x64 8w 32x32x16",   "direct 128x128x64 4w 16x16x32",
    "direct 256x128x64 4w 16x16x32",   "direct 128x256x64 4w 16x16x32",
    "direct 256x256x32 8w 32x32x16 s4", "direct 256x256x32 8w 32x32x16 s5",
    "direct 256x256x32 4w 32x32x16 s4", "direct 256x256x32 4w 32x32x16 s5",
    "direct 128x128x64 4w 16x16x32 s3", "direct 128x128x64 4w 16x16x32 s4",
    "direct 256x128x64 4w 32x32x16 s3", "direct 256x256x64 8w 32x32x16 prio",
    "direct 256x256x64 8w 32x32x16 ilv", "direct 256x256x64 8w 32x32x16 ilv+prio",
    "direct 256x256x64 8w 32x32x16 gm4", "direct 256x256x64 8w 32x32x16 gm16",
    "direct 256x256x64 4w 32x32x16 ilv+prio",
    "direct 256x256x64 8w 32x32x16 gm4 ilv spread",
    "direct 256x256x64 8w 32x32x16 gm4 ilv ntC",
    "direct 256x256x64 8w 32x32x16 gm4 ilv spread ntC",
    "direct 256x256x32 8w 32x32x16 s4 gm4 ilv ntC",
    "direct 256x256x64 4w 32x32x16 gm4 ilv+prio spread ntC",
    "direct 256x256x64 8w 16x16x32 gm4 ilv ntC agpr early"};
constexpr int kCount = sizeof(kNames) / sizeof(kNames[0]);

}  // namespace

int mfma16_config_count() { return kCount; }
const char* mfma16_config_name(int c) { return (c >= 0 && c < kCount) ? kNames[c] : nullptr; }

hipError_t launch_mfma16(const GemmArgs& g, int config) {
    return g.dtype == 1 ? launch_typed<_Float16>(g, config) : launch_typed<bf16_t>(g, config);
}

}  // namespace migemm
