// regtile_mfma_part.hip -- the kernels of one FP32 matrix-core configuration
// (see regtile_mfma.hip).  Built once per (output form, configuration): the
// build passes MIGEMM_PART_GEN (false: plain FP32 overwrite; true: the general
// output step) and MIGEMM_PART_C (the configuration index).
#include "mfma16_direct.hpp"

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
// direct-staged (global -> LDS without registers, mfma16_direct.hpp with 32-bit
// elements): <E, BM, BN, WM, WN, MF, STAGES, BK, GM, SCHED, FLAGS>; FLAGS 48: all
// operand layouts and K in whole 4-element chunks (a partial last k-tile is
// zero-filled), | 2: non-temporal C stores (chosen when C rows are whole lines)
using D8 = DirectCfg<float, 64, 64, 2, 4, 16, 4, 32, 8, 2, 178>;    // 8 waves of 32x16; split-K
using D8P = DirectCfg<float, 64, 64, 2, 4, 16, 4, 32, 8, 2, 176>;
using D9 = DirectCfg<float, 64, 64, 2, 2, 16, 4, 32, 8, 2, 50>;     // 4 waves of 32x32
using D9P = DirectCfg<float, 64, 64, 2, 2, 16, 4, 32, 8, 2, 48>;
using D10 = DirectCfg<float, 128, 128, 2, 4, 16, 4, 32, 4, 2, 50>;  // 8 waves of 64x32
using D10P = DirectCfg<float, 128, 128, 2, 4, 16, 4, 32, 4, 2, 48>;
using D11 = DirectCfg<float, 128, 64, 2, 4, 16, 4, 32, 8, 2, 50>;   // 8 waves of 64x16
using D11P = DirectCfg<float, 128, 64, 2, 4, 16, 4, 32, 8, 2, 48>;



// The direct-staged configuration (NT stores or plain) where its preconditions
// hold, else the register-staged configuration with index F.
template <class D, class DP, int F, bool GEN>
hipError_t direct_or(const GemmArgs& g) {
    if (!direct_fits<D>(g)) return launch_regtile_mfma(g, F);
    return c_whole_lines(g.out) ? launch_direct_cfg<D, GEN>(g) : launch_direct_cfg<DP, GEN>(g);
}

}  // namespace

template <bool GEN, int C>
hipError_t launch_f32_cfg(const GemmArgs& g) {
    if constexpr (C == 0) return launch_mfma_cfg<F0, GEN>(g);
    else if constexpr (C == 1) return launch_mfma_cfg<F1, GEN>(g);
    else if constexpr (C == 2) return launch_mfma_cfg<F2, GEN>(g);
    else if constexpr (C == 3) return launch_mfma_cfg<F3, GEN>(g);
    else if constexpr (C == 4) return launch_mfma_cfg<F4, GEN>(g);
    else if constexpr (C == 5) return launch_mfma_cfg<F5, GEN>(g);
    else if constexpr (C == 6) return launch_mfma_cfg<F6, GEN>(g);
    else if constexpr (C == 7) return launch_mfma_cfg<F7, GEN>(g);
    else if constexpr (C == 8) return direct_or<D8, D8P, 2, GEN>(g);
    else if constexpr (C == 9) return direct_or<D9, D9P, 2, GEN>(g);
    else if constexpr (C == 10) return direct_or<D10, D10P, 0, GEN>(g);
    else if constexpr (C == 11) return direct_or<D11, D11P, 4, GEN>(g);
    else
        static_assert(C == 0, "no such configuration");
}

#if defined(MIGEMM_PART_GEN) && defined(MIGEMM_PART_C)
template hipError_t launch_f32_cfg<MIGEMM_PART_GEN, MIGEMM_PART_C>(const GemmArgs&);
#else
#error "regtile_mfma_part.hip is built with MIGEMM_PART_GEN and MIGEMM_PART_C defined"
#endif

}  // namespace migemm
