// pack.hip -- FP16/BF16 products whose operands the direct-staged kernel cannot
// read in place, or reads slowly: a pointer off a 16-byte boundary, a leading
// dimension that is not a whole number of 16-byte chunks, a contiguous side (K
// of a row-major A or of B given transposed, N of row-major B, M of A given
// transposed) that ends inside a chunk, or k-contiguous rows that do not start
// on 128-byte lines (each 128-byte k-tile row would then span two lines).
//
// The product C = A x B (page "CUDA-Practice 09", the definition of the
// row-major product) does not depend on where the operands sit in memory, and
// padding the k sum with zeros adds nothing to it: each extra term is an exact
// zero product.  So each such operand is first copied into a workspace as a
// k-contiguous row image, A' (M x K) or B' (N x K, that is B transposed), rows
// starting on 128-byte lines (leading dimension K rounded up to 64) and
// zero-filled from K to the end of the row.  The direct kernel then multiplies the
// copies and any operand left in place with the call's own M and N, and K (K
// rounded up to 64 when both operands are copies): it clamps ragged M and N
// rows, zero-fills a partial last k-tile, and reads a copy's last chunk whole;
// the output step writes C exactly as for the unpacked call.
//
// The copy is memory-bound: 2 bytes read and 2 written per element copied,
// small beside the product for the shapes this path is selected for.  One
// launch copies both operands, a workgroup one 64 x 64 tile at a time.  An
// operand that is transposed on the way (or whose rows are not 16-byte
// aligned) goes through LDS, so that the reads (2 bytes per lane, any
// alignment) and the writes (16 bytes per lane) are contiguous across a
// wavefront in either orientation; one that keeps its orientation and has
// aligned rows is copied 16 bytes at a time.
//
// Workspace: each copied operand's rows x leading dimension x 2 bytes, A' first
// (rounded up to 256 bytes), lent by the caller for this one call and 256-byte
// aligned; the library allocates nothing and keeps no pointer to it.  Without a
// large enough workspace the product runs on the register-staged kernel
// instead, which reads any layout in place.

#include "common.hpp"

namespace migemm {
namespace {

constexpr int kTile = 64;

// One operand copy: dst (rows x cols_out, leading dimension ldd, rows on
// 128-byte lines) from src,
//   dst[r][c] = src(r, c) for c < cols, 0 for cols <= c < cols_out,
//   src(r, c) = trans ? src[c * lds + r] : src[r * lds + c].
struct PackJob {
    const uint16_t* src;
    int64_t lds, rows, cols;
    uint16_t* dst;
    int64_t ldd, cols_out, tiles_c, tiles;
    int trans;
    int vec;  // not transposed, rows 16-byte aligned: straight 16-byte copies
};

// Workgroups stride over the 64 x 64 tiles of both jobs (job 0's tiles first).
// Reads are 2-byte loads, a wavefront covering 128 contiguous source bytes
// (any alignment); writes are 16-byte stores of 8 consecutive dst columns.
//
// Tile order.  A source row whose start is not on a 128-byte line puts each
// 128-byte tile row across two lines, the second shared with the next tile
// along the source's contiguous side.  Consecutive tile indices therefore run
// along that side (dst rows for a transposed job, dst columns otherwise), and
// the workgroups of one XCD (blockIdx modulo 8) take one contiguous range of
// indices, so a shared line is fetched into that XCD's L2 once instead of into
// two XCDs' L2s.
__global__ __launch_bounds__(256) void pack16_kernel(PackJob j0, PackJob j1) {
    __shared__ uint32_t tile[kTile][kTile + 1];
    const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;   // reads: ty in 0..3
    const int wx = threadIdx.x % 8, wy = threadIdx.x / 8;           // writes: wy in 0..31
    const int64_t total = j0.tiles + j1.tiles;
    const int64_t per = gridDim.x / kNumXcd;
    const int64_t first = blockIdx.x < per * kNumXcd
                              ? (blockIdx.x % kNumXcd) * per + blockIdx.x / kNumXcd
                              : blockIdx.x;
    for (int64_t t = first; t < total; t += gridDim.x) {
        const bool second = t >= j0.tiles;
        const PackJob& j = second ? j1 : j0;
        const int64_t tt = second ? t - j0.tiles : t;
        const int64_t tiles_r = j.tiles / j.tiles_c;
        const int64_t r0 = (j.trans ? tt % tiles_r : tt / j.tiles_c) * kTile;
        const int64_t c0 = (j.trans ? tt / tiles_r : tt % j.tiles_c) * kTile;
        if (j.vec) {
            // 64 rows x 8 chunks of 16 bytes, two per work-item; the chunk that
            // straddles cols (cols not a multiple of 8) is read element by element
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int q = threadIdx.x + 256 * i;
                const int64_t r = r0 + q / 8, c = c0 + 8 * (q % 8);
                if (r >= j.rows || c >= j.cols_out) continue;
                u32x4 w = {0u, 0u, 0u, 0u};
                const uint16_t* s = j.src + r * j.lds + c;
                if (c + 8 <= j.cols) {
                    w = *reinterpret_cast<const u32x4*>(s);
                } else if (c < j.cols) {
                    for (int e = 0; e < 8 && c + e < j.cols; ++e)
                        w[e / 2] |= static_cast<uint32_t>(s[e]) << (16 * (e % 2));
                }
                *reinterpret_cast<u32x4*>(j.dst + r * j.ldd + c) = w;
            }
            continue;  // the whole workgroup takes this branch: no barrier is skipped
        }
        // tile[c - c0][r - r0] = src(r, c), zero outside the source.  Every
        // load reads a clamped in-bounds address and the zero is selected
        // afterwards, so the sixteen loads of a lane are in flight together.
        uint32_t v[kTile / 4];
        if (j.trans) {
            const int64_t r = r0 + tx, rc = r < j.rows ? r : j.rows - 1;
#pragma unroll
            for (int i = 0; i < kTile / 4; ++i) {
                const int64_t c = c0 + ty + 4 * i, cc = c < j.cols ? c : j.cols - 1;
                v[i] = j.src[cc * j.lds + rc];
            }
#pragma unroll
            for (int i = 0; i < kTile / 4; ++i) {
                const bool in = r < j.rows && c0 + ty + 4 * i < j.cols;
                tile[ty + 4 * i][tx] = in ? v[i] : 0u;
            }
        } else {
            const int64_t c = c0 + tx, cc = c < j.cols ? c : j.cols - 1;
#pragma unroll
            for (int i = 0; i < kTile / 4; ++i) {
                const int64_t r = r0 + ty + 4 * i, rc = r < j.rows ? r : j.rows - 1;
                v[i] = j.src[rc * j.lds + cc];
            }
#pragma unroll
            for (int i = 0; i < kTile / 4; ++i) {
                const bool in = r0 + ty + 4 * i < j.rows && c < j.cols;
                tile[tx][ty + 4 * i] = in ? v[i] : 0u;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kTile / 32; ++i) {
            const int rr = wy + 32 * i;
            const int64_t r = r0 + rr, c = c0 + 8 * wx;
            if (r < j.rows && c < j.cols_out) {  // cols_out is a multiple of 8
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = tile[8 * wx + 2 * e][rr] | (tile[8 * wx + 2 * e + 1][rr] << 16);
                *reinterpret_cast<u32x4*>(j.dst + r * j.ldd + c) = w;
            }
        }
        __syncthreads();
    }
}

int64_t round_up(int64_t x, int64_t m) { return ceil_div(x, m) * m; }

// Rows of dst start on 128-byte lines and are written whole (zero-filled from
// cols to the leading dimension), so every line of the copy is written in full.
PackJob make_job(const void* src, int64_t lds, int64_t rows, int64_t cols, bool trans, void* dst) {
    const int64_t ldd = round_up(cols, 64), cols_out = ldd;
    PackJob j;
    j.src = static_cast<const uint16_t*>(src);
    j.lds = lds;
    j.rows = rows;
    j.cols = cols;
    j.dst = static_cast<uint16_t*>(dst);
    j.ldd = ldd;
    j.cols_out = cols_out;
    j.tiles_c = ceil_div(cols_out, kTile);
    j.tiles = ceil_div(rows, kTile) * j.tiles_c;
    j.trans = trans ? 1 : 0;
    j.vec = !trans && aligned16(src) && lds % 8 == 0;
    return j;
}

hipError_t launch_pack16(const GemmArgs& g, const PackJob& j0, const PackJob& j1) {
    const int64_t tiles = j0.tiles + j1.tiles;
    if (tiles == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(tiles < 65536 ? tiles : 65536);
    return launch_kernel(g, pack16_kernel, dim3(grid), dim3(256), j0, j1);
}

// The direct configuration that packed configuration pc (11 or 12) runs.  11:
// the 256x256 ping-pong kernel on whole tiles and whole k-tiles (configuration
// 14), else the 256x256 interleaved one (10, which runs a partial first k-tile
// when K is whole 16-byte chunks), else the 128x256 one (13, which zero-fills a
// partial last k-tile and reads a copy's zero-filled last chunk).  12: the
// 128x128 one (7, with the partial last k-tile too).
int inner_config(const GemmArgs& g, int pc) {
    if (pc == 12) return 7;
    if (g.K % 64 != 0) return g.K % 8 == 0 ? 10 : 13;
    return (g.M % 256 == 0 && g.N % 256 == 0) ? 14 : 10;
}

// One operand's plan.  A row image (row-major A, B given transposed) is read in
// place when 16-byte aligned, K is whole chunks and its rows start on 128-byte
// lines; otherwise it is copied as it is.  A k-row image (A given transposed,
// row-major B) is read in place when 16-byte aligned with its side (M or N) in
// whole chunks; otherwise it is transposed into a row image.
struct Operand {
    bool in_place, trans;
    int64_t rows, bytes;  // rows: M or N
};

Operand plan_operand(const void* p, int64_t ld, int64_t rows, int64_t K, bool row_image) {
    Operand o;
    o.rows = rows;
    o.trans = !row_image;
    o.in_place = aligned16(p) && ld % 8 == 0 &&
                 (row_image ? (K % 8 == 0 && (ld * 2) % 128 == 0) : rows % 8 == 0);
    o.bytes = o.in_place ? 0 : rows * round_up(K, 64) * 2;
    return o;
}

struct PackPlan {
    int inner;
    Operand a, b;
    int64_t a_bytes;  // A' rounded up to the workspace alignment (B' follows it)
};

PackPlan plan_pack(const GemmArgs& g, int pc) {
    PackPlan p;
    p.inner = inner_config(g, pc);
    p.a = plan_operand(g.A, g.lda, g.M, g.K, !g.ta);
    p.b = plan_operand(g.B, g.ldb, g.N, g.K, g.tb);
    p.a_bytes = round_up(p.a.bytes, kWorkspaceAlign);
    return p;
}

}  // namespace

int64_t packed_k(int64_t K) { return ceil_div(K, 64) * 64; }

int64_t packed16_workspace_bytes(const GemmArgs& g, int pc) {
    const PackPlan p = plan_pack(g, pc);
    return p.b.bytes ? p.a_bytes + p.b.bytes : p.a.bytes;
}

bool packed16_workspace_ok(const GemmArgs& g, int pc) {
    return g.ws != nullptr && (reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign) == 0 &&
           g.ws_bytes >= packed16_workspace_bytes(g, pc);
}

hipError_t launch_packed16(const GemmArgs& g, int pc, int fallback_config) {
    const PackPlan pl = plan_pack(g, pc);
    if (pl.a.in_place && pl.b.in_place) return launch_mfma16(g, pl.inner);
    if (!packed16_workspace_ok(g, pc)) return launch_mfma16(g, fallback_config);
    char* const wa = static_cast<char*>(g.ws);
    char* const wb = wa + pl.a_bytes;
    // A' (M x K): row-major A is copied, A given transposed (K x M) is transposed.
    // B' (N x K): row-major B (K x N) is transposed, B given transposed is copied.
    const PackJob none = make_job(nullptr, 8, 0, 0, false, nullptr);
    const PackJob ja = pl.a.in_place ? none : make_job(g.A, g.lda, g.M, g.K, g.ta, wa);
    const PackJob jb = pl.b.in_place ? none : make_job(g.B, g.ldb, g.N, g.K, !g.tb, wb);
    hipError_t e = launch_pack16(g, ja, jb);
    if (e != hipSuccess) return e;
    GemmArgs p = g;
    // Both operands copies, zero-filled to K rounded up to 64: the product runs
    // on whole k-tiles, without the partial-k-tile instantiation.
    if (!pl.a.in_place && !pl.b.in_place) p.K = round_up(g.K, 64);
    if (!pl.a.in_place) {
        p.ta = false;
        p.A = wa;
        p.lda = ja.ldd;
        p.pad_a = true;
    }
    if (!pl.b.in_place) {
        p.tb = true;
        p.B = wb;
        p.ldb = jb.ldd;
        p.pad_b = true;
    }
    return launch_mfma16(p, pl.inner);
}

}  // namespace migemm
