// naive.hip -- one work-item per element of C, the in-repo baseline.
//
// Work-item (i, j) accumulates C[i][j] = sum_k A[i][k] * B[k][j] in FP32 with
// one fused multiply-add per k, reading A and B straight from global memory
// (page "04-wmma-matmul.cu", naiveMatmul; page "CUDA-Practice 09",
// gemm_fp32_kernel, which generalises it to M, N, K).  FP16 and BF16 inputs
// are widened exactly to FP32 before the multiply, so the mixed-precision
// semantics are those of the matrix-core kernels.
//
// Either operand may be given transposed: the kernel walks k with the
// operands' own strides (A: 1 or lda, B: ldb or 1).
//
// Launch shape for wave64: a 64 x 4 workgroup, so each wavefront covers 64
// consecutive columns of one row of C -- its B loads are one 256-byte
// coalesced read per k and its A load is a single broadcast address.  The
// pages' 16 x 16 block (which on wave64 would put 4 rows of 16 columns in one
// wavefront) is kept as configuration 1 for comparison.
#include "common.hpp"

namespace migemm {
namespace {

template <typename T, int BX, int BY, bool GEN>
__global__ __launch_bounds__(BX* BY) void naive_kernel(int64_t M, int64_t N, int64_t K,
                                                       const T* __restrict__ A, int64_t lda,
                                                       const T* __restrict__ B, int64_t ldb,
                                                       bool ta, bool tb, Epi out) {
    const int64_t col = static_cast<int64_t>(blockIdx.x) * BX + threadIdx.x;
    if (col >= N) return;
    // grid.y is capped at 65535 by the launcher; rows beyond it loop.
    for (int64_t row = static_cast<int64_t>(blockIdx.y) * BY + threadIdx.y; row < M;
         row += static_cast<int64_t>(gridDim.y) * BY) {
        const T* a = ta ? A + row : A + row * lda;
        const T* b = tb ? B + col * ldb : B + col;
        const int64_t sa = ta ? lda : 1, sb = tb ? 1 : ldb;  // step along k
        float acc = 0.0f;
        for (int64_t k = 0; k < K; ++k) acc = fmaf(to_f32(a[k * sa]), to_f32(b[k * sb]), acc);
        store_out<GEN>(out, row * out.ldc + col, acc);
    }
}

template <int BX, int BY, bool GEN>
hipError_t launch_shape(const GemmArgs& g) {
    const int64_t gy = ceil_div(g.M, BY);
    dim3 grid(static_cast<unsigned>(ceil_div(g.N, BX)),
              static_cast<unsigned>(gy > 65535 ? 65535 : gy));
    dim3 block(BX, BY);
    switch (g.dtype) {
        case 0:
            return launch_kernel(g, naive_kernel<float, BX, BY, GEN>, grid, block, g.M, g.N, g.K,
                                 static_cast<const float*>(g.A), g.lda,
                                 static_cast<const float*>(g.B), g.ldb, g.ta, g.tb, g.out);
        case 1:
            return launch_kernel(g, naive_kernel<_Float16, BX, BY, GEN>, grid, block, g.M, g.N,
                                 g.K, static_cast<const _Float16*>(g.A), g.lda,
                                 static_cast<const _Float16*>(g.B), g.ldb, g.ta, g.tb, g.out);
        default:
            return launch_kernel(g, naive_kernel<bf16_t, BX, BY, GEN>, grid, block, g.M, g.N,
                                 g.K, static_cast<const bf16_t*>(g.A), g.lda,
                                 static_cast<const bf16_t*>(g.B), g.ldb, g.ta, g.tb, g.out);
    }
}

const char* const kNames[] = {"64x4 wave-per-row", "16x16 square"};

}  // namespace

int naive_config_count() { return 2; }
const char* naive_config_name(int c) { return (c >= 0 && c < 2) ? kNames[c] : nullptr; }

hipError_t launch_naive(const GemmArgs& g, int config) {
    // The grid's x extent must fit 32 bits; N < 2^31 is checked by the caller.
    if (g.general()) return config == 1 ? launch_shape<16, 16, true>(g) : launch_shape<64, 4, true>(g);
    return config == 1 ? launch_shape<16, 16, false>(g) : launch_shape<64, 4, false>(g);
}

}  // namespace migemm
