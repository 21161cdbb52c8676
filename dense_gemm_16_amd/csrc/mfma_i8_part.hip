// mfma_i8_part.hip -- the kernels of one INT8 configuration (see mfma_i8.hip).
// Built once per configuration: the build passes MIGEMM_PART_C.
#include "mfma16_direct.hpp"

namespace migemm {

template <int C>
hipError_t launch_i8_cfg(const GemmArgs& g);

namespace {

using I0 = MfmaCfg<int8_t, 256, 256, 2, 4, 16>;  // 8 waves, 128x64 per wave
using I1 = MfmaCfg<int8_t, 128, 128, 2, 2, 16>;  // 4 waves, 64x64 per wave
using I2 = MfmaCfg<int8_t, 64, 64, 2, 2, 16>;    // small problems: 4x the workgroups
using I3 = MfmaCfg<int8_t, 256, 256, 2, 4, 32>;  // 8 waves, 32x32x32 instructions
// direct-staged ping-pong, whole tiles only, every layout; D4P with plain C
// stores for C rows that are not whole 128-byte lines
using D4 = DirectCfg<int8_t, 256, 256, 2, 4, 16, 2, 128, 4, 4, 22>;
using D4P = DirectCfg<int8_t, 256, 256, 2, 4, 16, 2, 128, 4, 4, 20>;
// direct-staged, interleaved schedule: any M and N (clamped loads, guarded
// stores), every layout, a partial first k-tile where K is not a multiple of
// 128; D6P with plain C stores
using D6 = DirectCfg<int8_t, 256, 256, 2, 4, 16, 2, 128, 4, 2, 222>;  // also split-K
using D6P = DirectCfg<int8_t, 256, 256, 2, 4, 16, 2, 128, 4, 2, 220>;

}  // namespace

template <int C>
hipError_t launch_i8_cfg(const GemmArgs& g) {
    if constexpr (C == 0) return launch_mfma_cfg<I0, false>(g);
    else if constexpr (C == 1) return launch_mfma_cfg<I1, false>(g);
    else if constexpr (C == 2) return launch_mfma_cfg<I2, false>(g);
    else if constexpr (C == 3) return launch_mfma_cfg<I3, false>(g);
    else if constexpr (C == 4)
        return !direct_fits<D4>(g)   ? launch_mfma_i8(g, 0)
               : c_whole_lines(g.out) ? launch_direct_cfg<D4, false>(g)
                                      : launch_direct_cfg<D4P, false>(g);
    else if constexpr (C == 6)
        return !direct_fits<D6>(g)   ? launch_mfma_i8(g, 3)
               : c_whole_lines(g.out) ? launch_direct_cfg<D6, false>(g)
                                      : launch_direct_cfg<D6P, false>(g);
    else
        static_assert(C == 0, "no such configuration");
}

#if defined(MIGEMM_PART_C)
template hipError_t launch_i8_cfg<MIGEMM_PART_C>(const GemmArgs&);
#else
#error "mfma_i8_part.hip is built with MIGEMM_PART_C defined"
#endif

}  // namespace migemm
