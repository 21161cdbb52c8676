// mfma16_general.hip -- the FP16/BF16 configurations compiled with the general
// output step: C = alpha * (sum of products) + beta * C_old, C in FP32, FP16
// or BF16 (the configuration table is in mfma16_configs.hpp).
#include "mfma16_configs.hpp"

namespace migemm {

hipError_t launch_mfma16_general(const GemmArgs& g, int config) {
    return g.dtype == 1 ? launch_typed<_Float16, true>(g, config)
                        : launch_typed<bf16_t, true>(g, config);
}

}  // namespace migemm
