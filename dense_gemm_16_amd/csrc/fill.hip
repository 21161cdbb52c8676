// fill.hip -- the product with K == 0: every sum of products is empty, so each
// element of the M x N window of C receives the output step applied to 0
// (C = 0 for the plain overwrite, C = beta C_old in general).  A kernel rather
// than a memset so that the padding between rows is left untouched and the
// call stays capturable.
#include "common.hpp"

namespace migemm {
namespace {

template <bool GEN>
__global__ __launch_bounds__(256) void empty_product_kernel(Epi out, int64_t M, int64_t N) {
    const int64_t total = M * N;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t r = e / N, c = e % N;
        store_out<GEN>(out, r * out.ldc + c, 0.0f);
    }
}

}  // namespace

hipError_t launch_empty_product(const GemmArgs& g) {
    int64_t blocks = ceil_div(g.M * g.N, 256);
    if (blocks > 65536) blocks = 65536;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    if (g.general()) return launch_kernel(g, empty_product_kernel<true>, grid, block, g.out, g.M, g.N);
    return launch_kernel(g, empty_product_kernel<false>, grid, block, g.out, g.M, g.N);
}

}  // namespace migemm
