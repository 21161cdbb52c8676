// splitk.hip -- products whose M x N is small beside K: the sum over k split
// into slices (FP16/BF16, FP32 and INT8).
//
// C = A x B (page "CUDA-Practice 09", the definition of the row-major product)
// is, element by element, the sum over k of A[i][k] B[k][j]; the sum splits
// into slices of k, each summed on its own and the slice sums added.  With
// 512 x 512 and K = 65536 the 128x128 tile gives 16 workgroups for 256 CUs, each
// walking all of K; as 16 slices of 4096 (whole 64-deep k-tiles, the last slice
// what is left) the same launch runs 256 workgroups, 16 per slice, each
// writing its FP32 sums plainly to its slice's M x N block of the caller's
// workspace.  A second kernel adds the slices of each element in slice order
// (so the result does not depend on timing) and applies the output step
// (alpha, beta, 16-bit C) to the total.  Both launch on the call's stream.
//
// The workgroups are renumbered so that each XCD takes whole slices: the tiles
// of one slice share its rows of A and columns of B in that XCD's L2, and each
// operand element is read from HBM about once (512 x 512 x 65536 BF16: 41 us,
// against 69 us with the slices spread over all eight XCDs and 217 us for the
// 64x64 tile without slices).
//
// FP16/BF16 split-K is used where a workspace is lent (slices x M x N x 4
// bytes), the operands suit the direct kernel, K is at least 6144 and
// 4 max(M, N), and the 128x128 tile would not fill a round of 256 workgroups.
// FP32 products slice on the 64x64 FP32 tile and INT8 ones on the interleaved
// 256x256 INT8 tile (INT32 sums, added exactly); their selection rules sit
// with the selection table.
#include "mfma16_configs.hpp"
#include "mfma16_direct.hpp"

namespace migemm {
namespace {

constexpr int kThreads = 256;

// INT32 slice sums of an INT8 product: out[idx] = the sum of part[s][idx] over
// the slices, written as INT32.  Each slice sum and the total are sums of at
// most K < 2^17 products of magnitude at most 2^14, below 2^31: every addition
// is exact, in any order.
template <int SMAX>
__global__ __launch_bounds__(kThreads) void splitk_reduce_i32(const int32_t* __restrict__ part,
                                                              int S, int64_t M, int64_t N,
                                                              Epi out) {
    const int64_t MN = M * N;
    const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 4;
    if (i0 >= MN) return;
    int32_t v[4] = {0, 0, 0, 0};
    if (i0 + 4 <= MN && MN % 4 == 0) {
        u32x4 p[SMAX];
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
            p[s] = *reinterpret_cast<const u32x4*>(part + (s < S ? s : S - 1) * MN + i0);
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            if (s < S) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += static_cast<int32_t>(p[s][e]);
            }
        }
    } else {
        for (int s = 0; s < S; ++s)
            for (int e = 0; i0 + e < MN && e < 4; ++e) v[e] += part[s * MN + i0 + e];
    }
    int32_t* const c = static_cast<int32_t*>(out.C);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + e;
        if (i < MN) c[(i / N) * out.ldc + i % N] = v[e];
    }
}

// out[idx] for 4 consecutive elements per work-item of the M x N result:
// the sum of part[s][idx], s = 0 .. S - 1 in order, then the output step.
// Every slice's 16 bytes are loaded before the first is added, so the S loads
// of a work-item are in flight together (one after another, S = 16 took 9.5 us
// for 16 MiB of sums); loads past the last slice read the last one again and
// are not added.  SMAX: S rounded up to 4, 8 or 16.
template <bool GEN, int SMAX>
__global__ __launch_bounds__(kThreads) void splitk_reduce(const float* __restrict__ part, int S,
                                                          int64_t M, int64_t N, Epi out) {
    const int64_t MN = M * N;
    const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 4;
    if (i0 >= MN) return;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (i0 + 4 <= MN && MN % 4 == 0) {  // 16-byte aligned in every slice
        f32x4 p[SMAX];
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
            p[s] = *reinterpret_cast<const f32x4*>(part + (s < S ? s : S - 1) * MN + i0);
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            if (s < S) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += p[s][e];
            }
        }
    } else {
        for (int s = 0; s < S; ++s)
            for (int e = 0; i0 + e < MN && e < 4; ++e) v[e] += part[s * MN + i0 + e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + e;
        if (i < MN) store_out<GEN>(out, (i / N) * out.ldc + i % N, v[e]);
    }
}

template <bool GEN>
hipError_t launch_reduce(const GemmArgs& g, int S, const float* part) {
    const dim3 grid(static_cast<unsigned>(ceil_div(ceil_div(g.M * g.N, 4), kThreads)));
    if (S <= 4)
        return launch_kernel(g, splitk_reduce<GEN, 4>, grid, dim3(kThreads), part, S, g.M, g.N,
                             g.out);
    if (S <= 8)
        return launch_kernel(g, splitk_reduce<GEN, 8>, grid, dim3(kThreads), part, S, g.M, g.N,
                             g.out);
    return launch_kernel(g, splitk_reduce<GEN, 16>, grid, dim3(kThreads), part, S, g.M, g.N,
                         g.out);
}

// Slices that, with `tiles` tiles each, make about one round of 256
// workgroups: 2 to 16.
int64_t round_slices(int64_t tiles) {
    const int64_t s = tiles > 0 ? 256 / tiles : 0;
    return s < 2 ? 2 : s > 16 ? 16 : s;
}

}  // namespace

// The tile and the slice count for this product.  The 128x128 tile
// (configuration 7) takes 2 to 16 slices, as many as make a round of 256
// workgroups.  The 256x256 tile (configuration 10) runs a 64-deep k-tile, four
// times the 128x128 tile's matrix work, in about 3 times its time (1.78 against
// 0.60 us), but as 4 times as many slices its FP32 sums cost 4 times the
// writes and reads; measured (BF16), it wins where its slices are at least
// 4096 deep (1024 x 1024 x 65536: 141.9 against 150.2 us; 2048 x 1024 x 65536:
// 243 against 308) and loses where they are 1024 or 2048 deep (1024 x 1024 x
// 16384: 53.9 against 40.1; 1024 x 1024 x 32768: 76.3 against 71.2).  It is
// also taken, with slices at least 1024 deep, where the 128x128 tile's two
// slices overshoot a round (more than 128 tiles: 1536 x 1536 x 8192, 56.6
// against 71.1 us).  Fewer slices where K runs out of whole k-tiles.
SplitKPlan splitk16_plan(const GemmArgs& g) {
    const int64_t t128 = ceil_div(g.M, 128) * ceil_div(g.N, 128);
    const int64_t t256 = ceil_div(g.M, 256) * ceil_div(g.N, 256);
    const int64_t s128 = round_slices(t128);
    if (t256 >= 16) {
        const int64_t ks = splitk_slice(g.K, round_slices(t256));
        if (ks >= kMinSlice256 || (t128 * s128 > 256 && ks >= kMinSlice256Overshoot))
            return SplitKPlan{10, ceil_div(g.K, ks)};
    }
    const int64_t ks = splitk_slice(g.K, s128);
    return SplitKPlan{7, ceil_div(g.K, ks)};
}

int64_t splitk16_slices(const GemmArgs& g) { return splitk16_plan(g).slices; }

// slices x M x N FP32 sums; 0 where split-K does not apply (fewer than two
// slices, or M x N beyond 2^30)
int64_t splitk16_workspace_bytes(const GemmArgs& g) {
    const int64_t s = splitk16_slices(g);
    if (s < 2 || g.M * g.N > (int64_t(1) << 30)) return 0;
    return s * g.M * g.N * 4;
}

template <bool GEN, int C>
hipError_t launch_f32_cfg(const GemmArgs& g);
template <int C>
hipError_t launch_i8_cfg(const GemmArgs& g);

int64_t splitk8_slices(const GemmArgs& g) {
    const int64_t ks =
        splitk_slice(g.K, round_slices(ceil_div(g.M, 256) * ceil_div(g.N, 256)), 128);
    return ceil_div(g.K, ks);
}

int64_t splitk8_workspace_bytes(const GemmArgs& g) {
    const int64_t s = splitk8_slices(g);
    if (s < 2 || g.M * g.N > (int64_t(1) << 30)) return 0;
    return s * g.M * g.N * 4;
}

hipError_t launch_splitk8(const GemmArgs& g) {
    const int64_t S = splitk8_slices(g), need = splitk8_workspace_bytes(g);
    if (need == 0 || S > 16 || g.ws == nullptr ||
        (reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign) != 0 || g.ws_bytes < need)
        return hipErrorInvalidValue;
    // the slices run on the interleaved direct kernel only (K whole 16-byte
    // chunks); other operands take the ordinary selection instead
    if (!direct_ok(g, 16, true, 16) || g.K % 16 != 0) return launch_mfma_i8(g, 3);
    GemmArgs p = g;
    p.splitk = static_cast<int>(S);
    p.out = Epi{g.ws, g.N, 1.0f, 0.0f, 4};  // INT32 slice sums, leading dimension N
    hipError_t e = launch_i8_cfg<6>(p);
    if (e != hipSuccess) return e;
    const int32_t* part = static_cast<const int32_t*>(g.ws);
    const dim3 grid(static_cast<unsigned>(ceil_div(ceil_div(g.M * g.N, 4), kThreads)));
    const int s = static_cast<int>(S);
    if (S <= 4)
        return launch_kernel(g, splitk_reduce_i32<4>, grid, dim3(kThreads), part, s, g.M, g.N,
                             g.out);
    if (S <= 8)
        return launch_kernel(g, splitk_reduce_i32<8>, grid, dim3(kThreads), part, s, g.M, g.N,
                             g.out);
    return launch_kernel(g, splitk_reduce_i32<16>, grid, dim3(kThreads), part, s, g.M, g.N,
                         g.out);
}

int64_t splitk32_slices(const GemmArgs& g) {
    const int64_t ks = splitk_slice(g.K, round_slices(ceil_div(g.M, 64) * ceil_div(g.N, 64)));
    return ceil_div(g.K, ks);
}

int64_t splitk32_workspace_bytes(const GemmArgs& g) {
    const int64_t s = splitk32_slices(g);
    if (s < 2 || g.M * g.N > (int64_t(1) << 30)) return 0;
    return s * g.M * g.N * 4;
}

hipError_t launch_splitk32(const GemmArgs& g) {
    const int64_t S = splitk32_slices(g), need = splitk32_workspace_bytes(g);
    if (need == 0 || S > 16 || g.ws == nullptr ||
        (reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign) != 0 || g.ws_bytes < need)
        return hipErrorInvalidValue;
    // the slices run on the direct kernel only (K whole 16-byte chunks of 4
    // elements); other operands take the ordinary 64x64 path instead
    if (!direct_ok(g, 4, true, 4)) return launch_regtile_mfma(g, 8);
    GemmArgs p = g;
    p.splitk = static_cast<int>(S);
    p.out = Epi{g.ws, g.N, 1.0f, 0.0f, 0};
    hipError_t e = launch_f32_cfg<false, 8>(p);
    if (e != hipSuccess) return e;
    const float* part = static_cast<const float*>(g.ws);
    return g.general() ? launch_reduce<true>(g, static_cast<int>(S), part)
                       : launch_reduce<false>(g, static_cast<int>(S), part);
}

hipError_t launch_splitk16(const GemmArgs& g) {
    const SplitKPlan plan = splitk16_plan(g);
    const int64_t S = plan.slices, need = splitk16_workspace_bytes(g);
    if (need == 0 || S > 16 || g.ws == nullptr ||
        (reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign) != 0 || g.ws_bytes < need)
        return hipErrorInvalidValue;
    // the slices run on the direct kernel only; operands it cannot read in
    // place take the ordinary 128x128 path instead
    if (!direct_ok(g, 8, true, 8) || g.K % 8 != 0) return launch_mfma16(g, 7);
    GemmArgs p = g;
    p.splitk = static_cast<int>(S);
    p.out = Epi{g.ws, g.N, 1.0f, 0.0f, 0};  // FP32 slice sums, plain, leading dimension N
    hipError_t e = launch_cfg16_any(p, plan.config);
    if (e != hipSuccess) return e;
    const float* part = static_cast<const float*>(g.ws);
    return g.general() ? launch_reduce<true>(g, static_cast<int>(S), part)
                       : launch_reduce<false>(g, static_cast<int>(S), part);
}

}  // namespace migemm
