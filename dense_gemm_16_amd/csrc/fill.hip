// fill.hip -- C = 0 over an M x N window with leading dimension ldc: the
// product with K == 0 (an empty sum).  A kernel rather than a memset so that
// the padding between rows is left untouched and the call stays capturable.
#include "common.hpp"

namespace migemm {
namespace {

__global__ __launch_bounds__(256) void zero_fill_kernel(float* __restrict__ C, int64_t M,
                                                        int64_t N, int64_t ldc) {
    const int64_t total = M * N;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t r = e / N, c = e % N;
        C[r * ldc + c] = 0.0f;
    }
}

}  // namespace

hipError_t launch_zero_fill(float* C, int64_t M, int64_t N, int64_t ldc, hipStream_t s) {
    int64_t blocks = ceil_div(M * N, 256);
    if (blocks > 65536) blocks = 65536;
    zero_fill_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(C, M, N, ldc);
    return hipGetLastError();
}

}  // namespace migemm
