// mfma16_configs.hpp -- the FP16/BF16 configuration table and its launcher,
// compiled once per output form: mfma16.hip for the plain FP32 overwrite,
// mfma16_general.hip for the general output step (alpha, beta, FP16/BF16 C).
// Two translation units keep each compile to one set of kernels and let the
// build run them in parallel.
#pragma once

#include "mfma16_direct.hpp"

namespace migemm {


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

template <class D, class Fallback, bool GEN>
hipError_t direct_or(const GemmArgs& g) {
    return direct_ok(g, D::BK) ? launch_direct_cfg<D, GEN>(g) : launch_mfma_cfg<Fallback, GEN>(g);
}

template <typename E, bool GEN>
hipError_t launch_typed(const GemmArgs& g, int config) {
    using T = Cfgs<E>;
    switch (config) {
        case 1: return launch_mfma_cfg<typename T::C1, GEN>(g);
        case 2: return launch_mfma_cfg<typename T::C2, GEN>(g);
        case 3: return launch_mfma_cfg<typename T::C3, GEN>(g);
        case 4: return launch_mfma_cfg<typename T::C4, GEN>(g);
        case 5: return launch_mfma_cfg<typename T::C5, GEN>(g);
        case 6: return launch_mfma_cfg<typename T::C6, GEN>(g);
        case 7: return direct_or<typename T::D7, typename T::C0, GEN>(g);
        case 8: return direct_or<typename T::D8, typename T::C0, GEN>(g);
        case 9: return direct_or<typename T::D9, typename T::C0, GEN>(g);
        case 10: return direct_or<typename T::D10, typename T::C0, GEN>(g);
        case 11: return direct_or<typename T::D11, typename T::C3, GEN>(g);
        case 12: return direct_or<typename T::D12, typename T::C2, GEN>(g);
        case 13: return direct_or<typename T::D13, typename T::C3, GEN>(g);
        case 14: return direct_or<typename T::D14, typename T::C0, GEN>(g);
        case 15: return direct_or<typename T::D15, typename T::C0, GEN>(g);
        case 16: return direct_or<typename T::D16, typename T::C0, GEN>(g);
        case 17: return direct_or<typename T::D17, typename T::C0, GEN>(g);
        case 18: return direct_or<typename T::D18, typename T::C3, GEN>(g);
        case 19: return direct_or<typename T::D19, typename T::C3, GEN>(g);
        case 20: return direct_or<typename T::D20, typename T::C2, GEN>(g);
        case 21: return direct_or<typename T::D21, typename T::C0, GEN>(g);
        case 22: return direct_or<typename T::D22, typename T::C0, GEN>(g);
        case 23: return direct_or<typename T::D23, typename T::C0, GEN>(g);
        case 24: return direct_or<typename T::D24, typename T::C0, GEN>(g);
        case 25: return direct_or<typename T::D25, typename T::C0, GEN>(g);
        case 26: return direct_or<typename T::D26, typename T::C0, GEN>(g);
        case 27: return direct_or<typename T::D27, typename T::C0, GEN>(g);
        case 28: return direct_or<typename T::D28, typename T::C0, GEN>(g);
        case 29: return direct_or<typename T::D29, typename T::C0, GEN>(g);
        case 30: return direct_or<typename T::D30, typename T::C0, GEN>(g);
        case 31: return direct_or<typename T::D31, typename T::C0, GEN>(g);
        case 32: return direct_or<typename T::D32, typename T::C0, GEN>(g);
        default: return launch_mfma_cfg<typename T::C0, GEN>(g);
    }
}

// The general output step over the same table (mfma16_general.hip).
hipError_t launch_mfma16_general(const GemmArgs& g, int config);

}  // namespace migemm
