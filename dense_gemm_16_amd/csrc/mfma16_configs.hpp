// mfma16_configs.hpp -- the FP16/BF16 configuration table's dispatch.  Each
// configuration is compiled on its own, once per element type and output form
// (mfma16_part.hip, built once per (type, form, configuration) so that the
// compiles run in parallel); mfma16.hip holds the names and the launcher.
#pragma once

#include "common.hpp"

namespace migemm {

// Configuration C of the table (indices as named in mfma16.hip) for element
// type E, with the plain FP32 overwrite (GEN false) or the general output step.
// Defined in mfma16_part.hip, explicitly instantiated there per part.
template <typename E, bool GEN, int C>
hipError_t launch_cfg16(const GemmArgs& g);

// Any configuration by index, for the element type and output form of g
// (mfma16.hip).  A direct-staged configuration whose preconditions do not hold
// calls this with its register-staged fallback's index.
hipError_t launch_cfg16_any(const GemmArgs& g, int config);

// Every configuration index that has a kernel of its own: the register-staged
// 0-4 and the direct-staged 5-10 and 13-16 (11 and 12 pack, then run one of
// these).
#define MIGEMM_CFG16_LIST(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) \
    X(13) X(14) X(15) X(16)

}  // namespace migemm
