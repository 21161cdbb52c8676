// mfma_i8.hip -- INT8 inputs, exact INT32 sums, on the gfx950 integer matrix-core
// instructions (v_mfma_i32_16x16x64_i8, v_mfma_i32_32x32x32_i8): configuration
// names and dispatch (the kernels of each configuration are compiled in
// mfma_i8_part.hip, one object per configuration).
//
// The tiled matrix-unit algorithm of page "Tensor cores and matrix operations"
// (section "Complete Algorithm for Large Matrix Multiply") on 8-bit operands:
// the register-staged pipeline of mfma_gemm.hpp with 16-element (16-byte)
// chunks, so a k-tile is 128 deep and one instruction consumes one chunk of A
// and of B per lane (16 k).  Operands whose M or N side is contiguous (row-major
// B, or A given transposed) are transposed in registers as 16 x 16 byte blocks.
// Every product of two int8 values is at most 2^14 in magnitude, so a sum of at
// most 2^17 - 1 of them is below 2^31 and the INT32 result is exact (the C ABI
// limits K to 2^17 - 1 for this type); C is written as INT32.
//
// Configuration 4 is the direct-staged ping-pong kernel of mfma16_direct.hpp on
// 8-bit elements: a 128-deep k-tile is a 128-byte row of A and a 256-byte k-row
// of B, as wide in bytes as the 64-deep 16-bit k-tile, so the LDS stages, the
// schedule and the 16-byte fragments carry over; row-major B is transposed by
// 8-bit transposing LDS reads.  It needs whole 256 x 256 tiles, K a multiple of
// 128, 16-byte aligned operands and leading dimensions in whole 16-byte chunks;
// other shapes run configuration 0.  Configuration 6 is the interleaved direct
// kernel on 8-bit elements (any M and N, K a multiple of 16), 5 copies operands
// the direct kernels cannot read (pack.hip), and 7 sums slices of K (splitk.hip).
#include "common.hpp"

namespace migemm {

template <int C>
hipError_t launch_i8_cfg(const GemmArgs& g);

namespace {

const char* const kNames[] = {"256x256x128 8w 16x16x64", "128x128x128 4w 16x16x64",
                              "64x64x128 4w 16x16x64", "256x256x128 8w 32x32x32",
                              "direct 256x256x128 8w 16x16x64 gm4 pingpong ntC agpr",
                              "packed: aligned zero-padded copies, then config 4, 3, 6, 1 or 2",
                              "direct 256x256x128 8w 16x16x64 gm4 ilv ntC agpr early",
                              "split-K: slices of K on config 6 into INT32 partials in the "
                              "workspace, then their sum"};
constexpr int kCount = sizeof(kNames) / sizeof(kNames[0]);

}  // namespace

int mfma_i8_config_count() { return kCount; }
const char* mfma_i8_config_name(int c) { return (c >= 0 && c < kCount) ? kNames[c] : nullptr; }

namespace {

hipError_t launch_cfg(const GemmArgs& g, int config) {
    switch (config) {
        case 1: return launch_i8_cfg<1>(g);
        case 2: return launch_i8_cfg<2>(g);
        case 3: return launch_i8_cfg<3>(g);
        case 4: return launch_i8_cfg<4>(g);
        case 6: return launch_i8_cfg<6>(g);
        default: return launch_i8_cfg<0>(g);
    }
}

}  // namespace

// Ragged shapes (split.cpp).  The direct ping-pong kernel (configuration 4)
// takes whole 256x256 tiles only, and a shape with a partial last band of rows
// or columns otherwise runs entirely on the register-staged 256x256 kernel
// (configuration 3), 2.6 to 3.7 times slower at 8200 x 8192 x 8192 and 4100 x
// 4096 x 4096.  So when the operands suit the direct kernel, the whole tiles
// run on it and the rows and columns past them follow: up to 16 on the skinny
// kernel, more on the 64x64 tile (configuration 2).  The 128x128 and 256x256
// register-staged tiles split a last band that would start a round of its own,
// as the other element types do; the 64x64 tile only for tails of up to 16.
hipError_t launch_mfma_i8(const GemmArgs& g, int config) {
    if (config == 5) return launch_packed8(g);
    if (config == 7) {
        // without a usable workspace the configuration the selection gives
        const int64_t need = splitk8_workspace_bytes(g);
        if (need == 0 || g.ws == nullptr ||
            (reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign) != 0 || g.ws_bytes < need) {
            const bool aligned = aligned16(g.A) && aligned16(g.B) && g.lda % 16 == 0 &&
                                 g.ldb % 16 == 0;
            return launch_mfma_i8(g, i8_select(g.M, g.N, g.K, aligned && g.K % 128 == 0,
                                               aligned && g.K % 16 == 0));
        }
        return launch_splitk8(g);
    }
    if (config == 3 || config == 4) {
        const bool direct = g.K % 128 == 0 && aligned16(g.A) && aligned16(g.B) &&
                            g.lda % 16 == 0 && g.ldb % 16 == 0;
        SplitPlan p;
        p.m_main = g.M / 256 * 256;
        p.n_main = g.N / 256 * 256;
        p.rows = p.m_main > 0 && p.m_main < g.M;
        p.cols = p.n_main > 0 && p.n_main < g.N;
        if (direct && p.m_main > 0 && p.n_main > 0 && (p.rows || p.cols)) {
            if (!p.rows) p.m_main = g.M;
            if (!p.cols) p.n_main = g.N;
            return launch_split(g, p, launch_cfg, 4, launch_cfg, 2);
        }
    }
    if (config <= 3 && config != 2) {
        const int64_t t = config == 1 ? 128 : 256;
        const SplitPlan p = plan_split(g.M, g.N, t, t, int64_t(1) << 62);
        if (p.rows || p.cols) return launch_split(g, p, launch_cfg, config, launch_cfg, 2);
    } else if (config == 2) {
        const SplitPlan p = plan_split(g.M, g.N, 64, 64, 16);
        if (p.rows || p.cols) return launch_split(g, p, launch_cfg, 2, launch_cfg, 2);
    }
    return launch_cfg(g, config);
}

}  // namespace migemm
