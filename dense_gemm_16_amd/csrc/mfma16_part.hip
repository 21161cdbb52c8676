// mfma16_part.hip -- the kernels of the FP16/BF16 configuration table.
//
// Built once per (element type, output form, configuration): the build passes
// MIGEMM_PART_E (_Float16 or bf16_t), MIGEMM_PART_GEN (false: plain FP32
// overwrite of C; true: the general output step) and MIGEMM_PART_C (the
// configuration index), and each object holds that one configuration's
// kernels.  The register-staged fallback of a direct-staged configuration is
// reached through launch_cfg16_any, so no kernel is compiled twice.
#include "mfma16_configs.hpp"
#include "mfma16_direct.hpp"

namespace migemm {
namespace {

template <typename E> struct Cfgs {
    // register-staged: any shape, leading dimension and alignment
    using R0 = MfmaCfg<E, 256, 256, 2, 4, 16>;  // 8 waves, 128x64 per wave
    using R1 = MfmaCfg<E, 256, 128, 2, 2, 16>;  // 4 waves, 128x64 per wave
    using R2 = MfmaCfg<E, 128, 128, 2, 2, 16>;  // 4 waves, 64x64 per wave
    using R3 = MfmaCfg<E, 64, 64, 2, 2, 16>;    // 4 waves, 32x32 per wave
    using R4 = MfmaCfg<E, 256, 256, 2, 4, 32>;  // 8 waves, 32x32x16 instructions
    // direct-staged: <E, BM, BN, WM, WN, MF, STAGES, BK, GM, SCHED, FLAGS>
    using D5 = DirectCfg<E, 256, 256, 2, 4, 16, 2, 64>;
    using D6 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64>;
    using D7 = DirectCfg<E, 128, 128, 2, 4, 16, 4, 64, 4, 2, 178>;  // 8 waves, interleave, gm4, nt C; all layouts; ragged K; split-K
    using D7P = DirectCfg<E, 128, 128, 2, 4, 16, 4, 64, 4, 2, 176>; // D7 with plain C stores
    using D8 = DirectCfg<E, 128, 128, 2, 2, 16, 4, 64>;             // 4 waves, 4 stages
    using D9 = DirectCfg<E, 256, 256, 2, 4, 32, 2, 64, 4, 2, 2>;    // gm4, interleave, nt C
    using D10 = DirectCfg<E, 256, 256, 2, 4, 16, 2, 64, 4, 2, 222>; // + AGPRs, early loads; all layouts; partial first k-tile; split-K
    using D10P = DirectCfg<E, 256, 256, 2, 4, 16, 2, 64, 4, 2, 220>; // D10 with plain C stores
    using D13 = DirectCfg<E, 128, 256, 2, 4, 16, 3, 64, 8, 2, 48>;  // 8 waves of 64x64, 3 stages; all layouts; ragged K
    using D14 = DirectCfg<E, 256, 256, 2, 4, 16, 2, 64, 4, 4, 22>;  // ping-pong (whole tiles), AGPRs, nt C; all layouts
    using D14P = DirectCfg<E, 256, 256, 2, 4, 16, 2, 64, 4, 4, 20>; // D14 with plain C stores
    using D15 = DirectCfg<E, 128, 256, 2, 4, 16, 2, 64, 8, 4, 22>;  // ping-pong 128x256 (whole tiles); all layouts
    using D15P = DirectCfg<E, 128, 256, 2, 4, 16, 2, 64, 8, 4, 20>; // D15 with plain C stores
    using D16 = DirectCfg<E, 64, 64, 2, 4, 16, 4, 64, 8, 0, 58>;    // 8 waves of 32x16, 4 stages, early loads, nt C; all layouts; ragged K
    using D16P = DirectCfg<E, 64, 64, 2, 4, 16, 4, 64, 8, 0, 56>;   // D16 with plain C stores
};

// The direct-staged configuration D where its preconditions hold, else the
// register-staged configuration with index F.
template <class D, int F, bool GEN>
hipError_t direct_or(const GemmArgs& g) {
    return direct_fits<D>(g) ? launch_direct_cfg<D, GEN>(g) : launch_cfg16_any(g, F);
}

}  // namespace

template <typename E, bool GEN, int C>
hipError_t launch_cfg16(const GemmArgs& g) {
    using T = Cfgs<E>;
    if constexpr (C == 0) return launch_mfma_cfg<typename T::R0, GEN>(g);
    else if constexpr (C == 1) return launch_mfma_cfg<typename T::R1, GEN>(g);
    else if constexpr (C == 2) return launch_mfma_cfg<typename T::R2, GEN>(g);
    else if constexpr (C == 3) return launch_mfma_cfg<typename T::R3, GEN>(g);
    else if constexpr (C == 4) return launch_mfma_cfg<typename T::R4, GEN>(g);
    else if constexpr (C == 5) return direct_or<typename T::D5, 0, GEN>(g);
    else if constexpr (C == 6) return direct_or<typename T::D6, 0, GEN>(g);
    else if constexpr (C == 7)
        return c_whole_lines(g.out) ? direct_or<typename T::D7, 2, GEN>(g)
                                    : direct_or<typename T::D7P, 2, GEN>(g);
    else if constexpr (C == 8) return direct_or<typename T::D8, 2, GEN>(g);
    else if constexpr (C == 9) return direct_or<typename T::D9, 0, GEN>(g);
    else if constexpr (C == 10)
        return c_whole_lines(g.out) ? direct_or<typename T::D10, 0, GEN>(g)
                                    : direct_or<typename T::D10P, 0, GEN>(g);
    else if constexpr (C == 13) return direct_or<typename T::D13, 2, GEN>(g);
    else if constexpr (C == 14)
        return c_whole_lines(g.out) ? direct_or<typename T::D14, 0, GEN>(g)
                                    : direct_or<typename T::D14P, 0, GEN>(g);
    else if constexpr (C == 15)
        return c_whole_lines(g.out) ? direct_or<typename T::D15, 2, GEN>(g)
                                    : direct_or<typename T::D15P, 2, GEN>(g);
    else if constexpr (C == 16)
        return c_whole_lines(g.out) ? direct_or<typename T::D16, 3, GEN>(g)
                                    : direct_or<typename T::D16P, 3, GEN>(g);
    else
        static_assert(C == 0, "no such configuration");
}

#if defined(MIGEMM_PART_E) && defined(MIGEMM_PART_GEN) && defined(MIGEMM_PART_C)
template hipError_t launch_cfg16<MIGEMM_PART_E, MIGEMM_PART_GEN, MIGEMM_PART_C>(const GemmArgs&);
#else
#error "mfma16_part.hip is built with MIGEMM_PART_E, MIGEMM_PART_GEN and MIGEMM_PART_C defined"
#endif

}  // namespace migemm
