// split.cpp -- running a tiled product as its whole tiles plus the ragged last
// band of rows and of columns.
//
// A tile-per-workgroup launch takes ceil(M / bm) x ceil(N / bn) workgroups in
// rounds of 256 (one per CU).  A few rows or columns past a whole number of
// tile bands can push that count just past a round, and the extra round costs
// as much as a full one while it runs a handful of tiles: 4100 x 4096 on 256x256
// tiles is 272 tiles, two rounds instead of one.  The same product (page
// "CUDA-Practice 09", the definition of the row-major product: every element of
// C is its own dot product) is then computed in pieces that each write their
// own part of C:
// * the whole tiles, rows [0, m_main) x columns [0, n_main), on the tile shape
//   that was asked for;
// * the rows past them, [m_main, M) x every column: up to 16 rows on the skinny
//   kernel, which spreads K over the waves of each workgroup, more on a smaller
//   tile;
// * the columns past them, [0, m_main) x [n_main, N) (every row when the rows are
//   not split): up to 16 columns as the transposed product C^T = B^T A^T on the
//   skinny kernel, written transposed into C, more on a smaller tile.
// The pieces run one after another on the call's stream.
#include "common.hpp"
#include "migemm.h"

namespace migemm {

namespace {

constexpr int64_t kCus = 256;

// Bytes per element of A and B (FP32, FP16/BF16, INT8) and of C (FP32 or INT32,
// FP16/BF16).
int64_t elem_bytes(int dtype) {
    return dtype == MIGEMM_F32 ? 4 : dtype == MIGEMM_I8 ? 1 : 2;
}
int64_t c_bytes(int c_dtype) {
    return (c_dtype == MIGEMM_F16 || c_dtype == MIGEMM_BF16) ? 2 : 4;
}

}  // namespace

SplitPlan plan_split(int64_t M, int64_t N, int64_t bm, int64_t bn, int64_t max_tail) {
    // whole and all tile rows (columns); split the rows, the columns or both,
    // whichever leaves the fewest rounds (fewer splits on a tie)
    const int64_t fm = M / bm, cm = ceil_div(M, bm), fn = N / bn, cn = ceil_div(N, bn);
    const bool can_m = fm > 0 && fm < cm && M - fm * bm <= max_tail;
    const bool can_n = fn > 0 && fn < cn && N - fn * bn <= max_tail;
    int64_t best = ceil_div(cm * cn, kCus);
    SplitPlan p;
    auto consider = [&](bool m, bool n) {
        if ((m && !can_m) || (n && !can_n)) return;
        const int64_t r = ceil_div((m ? fm : cm) * (n ? fn : cn), kCus);
        if (r < best) {
            best = r;
            p.rows = m;
            p.cols = n;
        }
    };
    consider(true, false);
    consider(false, true);
    consider(true, true);
    p.m_main = p.rows ? fm * bm : M;
    p.n_main = p.cols ? fn * bn : N;
    return p;
}

int f32_direct_tile(int64_t M, int64_t N) {
    // The 128x128 FP32 tile holds its CU alone (128 KiB of LDS); the 64x64 one runs
    // two workgroups per CU at about the same rate per multiply-add, so one of its
    // rounds (2 x 256 workgroups) is half the work of a 128x128 round.  The larger
    // tile is kept when it fills a round and, after the ragged last bands are split
    // off as the launch will do, needs at most half the smaller tile's rounds.
    if (ceil_div(M, 128) * ceil_div(N, 128) < kCus) return 8;
    auto rounds = [&](int64_t t, int64_t max_tail, int64_t slots) {
        const SplitPlan p = plan_split(M, N, t, t, max_tail);
        return ceil_div(ceil_div(p.m_main, t) * ceil_div(p.n_main, t), slots);
    };
    return 2 * rounds(128, 128, kCus) <= rounds(64, 16, 2 * kCus) ? 10 : 8;
}

hipError_t launch_split(const GemmArgs& g, const SplitPlan& p, CfgLauncher head, int head_config,
                        CfgLauncher tail, int tail_config) {
    const int64_t ea = elem_bytes(g.dtype), ec = c_bytes(g.out.c_dtype);
    GemmArgs h = g;
    h.M = p.m_main;
    h.N = p.n_main;
    hipError_t e = head(h, head_config);
    if (e != hipSuccess) return e;
    if (p.rows) {
        // rows [m_main, M), every column; row m_main of A is a column offset when
        // A is given transposed (K x M)
        GemmArgs t = g;
        t.M = g.M - p.m_main;
        t.A = static_cast<const char*>(g.A) + (g.ta ? p.m_main : p.m_main * g.lda) * ea;
        t.out.C = static_cast<char*>(g.out.C) + p.m_main * g.out.ldc * ec;
        e = skinny_fits(t) ? launch_skinny(t) : tail(t, tail_config);
        if (e != hipSuccess) return e;
    }
    if (p.cols) {
        // columns [n_main, N) of rows [0, m_main)
        const char* const bslab =
            static_cast<const char*>(g.B) + (g.tb ? p.n_main * g.ldb : p.n_main) * ea;
        char* const cslab = static_cast<char*>(g.out.C) + p.n_main * ec;
        if (g.N - p.n_main <= 16) {
            // C^T = B^T A^T: B's column slab is the left operand (k-contiguous
            // rows when B is given transposed or is a packed copy, k-rows
            // otherwise), A the right one
            GemmArgs t = g;
            t.M = g.N - p.n_main;
            t.N = p.m_main;
            t.A = bslab;
            t.ta = !g.tb;
            t.lda = g.ldb;
            t.pad_a = g.pad_b;
            t.B = g.A;
            t.tb = !g.ta;
            t.ldb = g.lda;
            t.pad_b = g.pad_a;
            t.out.C = cslab;
            t.trans_c = true;
            if (skinny_fits(t)) return launch_skinny(t);
        }
        GemmArgs t = g;
        t.M = p.m_main;
        t.N = g.N - p.n_main;
        t.B = bslab;
        t.out.C = cslab;
        return tail(t, tail_config);
    }
    return hipSuccess;
}

}  // namespace migemm
