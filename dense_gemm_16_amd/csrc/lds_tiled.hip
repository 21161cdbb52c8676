// lds_tiled.hip -- FP32 GEMM with square tiles of A and B staged in LDS.
//
// Per k-tile the workgroup copies a T x T tile of A and of B from global
// memory into LDS with coalesced loads (consecutive work-items take
// consecutive columns), waits at a barrier, lets every work-item accumulate
// its one output over the T values of k from LDS, and waits again before the
// tile is overwritten (page "matmul_registers.cu", matmulSharedTiled: two LDS
// reads per multiply-add, two barriers per k-tile).  Unlike that kernel this
// one guards every edge: out-of-range elements of A and B are loaded as zero
// and out-of-range outputs are not stored, so any M, N, K and leading
// dimension is accepted.
//
// LDS bank conflicts: a wavefront covers 64 / T rows of the tile, and its
// work-items read A_s[row][p] for those rows at once.  Rows of T floats map
// onto the same banks whenever T divides the bank count, so the tile rows are
// padded to T + 1 floats.  B_s[p][col] is read along a row, conflict-free.
//
// An operand given transposed (A stored K x M, B stored N x K) is read with
// the work-item's x index running along its contiguous side, so global reads
// stay coalesced, and written to LDS transposed (the padding keeps those
// column writes conflict-free).
#include "common.hpp"

namespace migemm {
namespace {

template <int T, bool GEN, bool TA, bool TB>
__global__ __launch_bounds__(T* T) void lds_tiled_kernel(int64_t M, int64_t N, int64_t K,
                                                        const float* __restrict__ A, int64_t lda,
                                                        const float* __restrict__ B, int64_t ldb,
                                                        Epi out) {
    __shared__ float As[T][T + 1];
    __shared__ float Bs[T][T + 1];
    const int tx = threadIdx.x, ty = threadIdx.y;
    const int64_t col = static_cast<int64_t>(blockIdx.x) * T + tx;
    const int64_t nrb = ceil_div(M, T);
    for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {  // uniform over the workgroup
        const int64_t row = rb * T + ty;
        float acc = 0.0f;
        for (int64_t k0 = 0; k0 < K; k0 += T) {
            if constexpr (TA) {  // element (rb*T + tx, k0 + ty), stored at A[k * lda + i]
                const int64_t i = rb * T + tx, k = k0 + ty;
                As[tx][ty] = (i < M && k < K) ? A[k * lda + i] : 0.0f;
            } else {
                const int64_t k = k0 + tx;
                As[ty][tx] = (row < M && k < K) ? A[row * lda + k] : 0.0f;
            }
            if constexpr (TB) {  // element (k0 + tx, blockIdx.x*T + ty), stored at B[j * ldb + k]
                const int64_t k = k0 + tx, j = static_cast<int64_t>(blockIdx.x) * T + ty;
                Bs[tx][ty] = (k < K && j < N) ? B[j * ldb + k] : 0.0f;
            } else {
                const int64_t k = k0 + ty;
                Bs[ty][tx] = (k < K && col < N) ? B[k * ldb + col] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int p = 0; p < T; ++p) acc = fmaf(As[ty][p], Bs[p][tx], acc);
            __syncthreads();
        }
        if (row < M && col < N) store_out<GEN>(out, row * out.ldc + col, acc);
    }
}

template <int T, bool GEN, bool TA, bool TB>
hipError_t launch_layout(const GemmArgs& g) {
    const int64_t gy = ceil_div(g.M, T);
    dim3 grid(static_cast<unsigned>(ceil_div(g.N, T)),
              static_cast<unsigned>(gy > 65535 ? 65535 : gy));
    return launch_kernel(g, lds_tiled_kernel<T, GEN, TA, TB>, grid, dim3(T, T), g.M, g.N, g.K,
                         static_cast<const float*>(g.A), g.lda, static_cast<const float*>(g.B),
                         g.ldb, g.out);
}

template <int T, bool GEN>
hipError_t launch_tile(const GemmArgs& g) {
    if (g.ta) return g.tb ? launch_layout<T, GEN, true, true>(g) : launch_layout<T, GEN, true, false>(g);
    return g.tb ? launch_layout<T, GEN, false, true>(g) : launch_layout<T, GEN, false, false>(g);
}

const char* const kNames[] = {"32x32 tile", "16x16 tile"};

}  // namespace

int lds_tiled_config_count() { return 2; }
const char* lds_tiled_config_name(int c) { return (c >= 0 && c < 2) ? kNames[c] : nullptr; }

hipError_t launch_lds_tiled(const GemmArgs& g, int config) {
    if (g.general()) return config == 1 ? launch_tile<16, true>(g) : launch_tile<32, true>(g);
    return config == 1 ? launch_tile<16, false>(g) : launch_tile<32, false>(g);
}

}  // namespace migemm
