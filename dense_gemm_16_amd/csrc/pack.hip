// pack.hip -- FP16/BF16 products (and, at the end of this file, INT8 ones)
// whose operands the direct-staged kernel cannot read in place, or reads
// slowly: a pointer off a 16-byte boundary, a leading
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
    const void* src;
    int64_t lds, rows, cols;
    void* dst;
    int64_t ldd, cols_out, tiles_c, tiles;
    int trans;
    int vec;  // not transposed, rows 16-byte aligned: straight 16-byte copies
};

// Workgroups stride over the 64 x 64 tiles of both jobs (job 0's tiles first).
// T is the element (uint16_t for FP16/BF16, uint8_t for INT8).  Reads are
// element loads, a wavefront covering 64 contiguous source elements (any
// alignment); writes are 16-byte stores of EPC = 16 / sizeof(T) consecutive
// dst columns.
//
// Tile order.  A source row whose start is not on a 128-byte line puts each
// 128-byte tile row across two lines, the second shared with the next tile
// along the source's contiguous side.  Consecutive tile indices therefore run
// along that side (dst rows for a transposed job, dst columns otherwise), and
// the workgroups of one XCD (blockIdx modulo 8) take one contiguous range of
// indices, so a shared line is fetched into that XCD's L2 once instead of into
// two XCDs' L2s.
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(PackJob j0, PackJob j1) {
    constexpr int EPC = 16 / sizeof(T);       // elements per 16-byte chunk: 8 or 16
    constexpr int CPR = kTile / EPC;          // chunks per tile row: 8 or 4
    constexpr int RPP = 256 / CPR;            // tile rows per pass of 256 work-items
    constexpr int PER = 4 / sizeof(T);        // elements per 32-bit word
    constexpr int BITS = 8 * sizeof(T);
    __shared__ uint32_t tile[kTile][kTile + 1];
    const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;   // reads: ty in 0..3
    const int wx = threadIdx.x % CPR, wy = threadIdx.x / CPR;       // writes: wy < RPP
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
        const T* const src = static_cast<const T*>(j.src);
        T* const dst = static_cast<T*>(j.dst);
        if (j.vec) {
            // 64 rows x CPR chunks of 16 bytes, 64 / RPP per work-item; the chunk
            // that straddles cols (cols not a multiple of EPC) is read element by
            // element
#pragma unroll
            for (int i = 0; i < kTile / RPP; ++i) {
                const int q = threadIdx.x + 256 * i;
                const int64_t r = r0 + q / CPR, c = c0 + EPC * (q % CPR);
                if (r >= j.rows || c >= j.cols_out) continue;
                u32x4 w = {0u, 0u, 0u, 0u};
                const T* s = src + r * j.lds + c;
                if (c + EPC <= j.cols) {
                    w = *reinterpret_cast<const u32x4*>(s);
                } else if (c < j.cols) {
                    for (int e = 0; e < EPC && c + e < j.cols; ++e)
                        w[e / PER] |= static_cast<uint32_t>(s[e]) << (BITS * (e % PER));
                }
                *reinterpret_cast<u32x4*>(dst + r * j.ldd + c) = w;
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
                v[i] = src[cc * j.lds + rc];
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
                v[i] = src[rc * j.lds + cc];
            }
#pragma unroll
            for (int i = 0; i < kTile / 4; ++i) {
                const bool in = r0 + ty + 4 * i < j.rows && c < j.cols;
                tile[tx][ty + 4 * i] = in ? v[i] : 0u;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kTile / RPP; ++i) {
            const int rr = wy + RPP * i;
            const int64_t r = r0 + rr, c = c0 + EPC * wx;
            if (r < j.rows && c < j.cols_out) {  // cols_out is a multiple of EPC
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t word = 0u;
#pragma unroll
                    for (int b = 0; b < PER; ++b) word |= tile[EPC * wx + PER * e + b][rr] << (BITS * b);
                    w[e] = word;
                }
                *reinterpret_cast<u32x4*>(dst + r * j.ldd + c) = w;
            }
        }
        __syncthreads();
    }
}

int64_t round_up(int64_t x, int64_t m) { return ceil_div(x, m) * m; }

// Rows of dst start on 128-byte lines and are written whole (zero-filled from
// cols to the leading dimension, cols rounded up to 128 bytes of es-byte
// elements), so every line of the copy is written in full.
PackJob make_job(const void* src, int64_t lds, int64_t rows, int64_t cols, bool trans, void* dst,
                 int es) {
    const int64_t ldd = round_up(cols, 128 / es), cols_out = ldd;
    PackJob j;
    j.src = src;
    j.lds = lds;
    j.rows = rows;
    j.cols = cols;
    j.dst = dst;
    j.ldd = ldd;
    j.cols_out = cols_out;
    j.tiles_c = ceil_div(cols_out, kTile);
    j.tiles = ceil_div(rows, kTile) * j.tiles_c;
    j.trans = trans ? 1 : 0;
    j.vec = !trans && aligned16(src) && lds % (16 / es) == 0;
    return j;
}

hipError_t launch_pack(const GemmArgs& g, const PackJob& j0, const PackJob& j1, int es) {
    const int64_t tiles = j0.tiles + j1.tiles;
    if (tiles == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(tiles < 65536 ? tiles : 65536);
    if (es == 1) return launch_kernel(g, pack_kernel<uint8_t>, dim3(grid), dim3(256), j0, j1);
    if (es == 4) return launch_kernel(g, pack_kernel<uint32_t>, dim3(grid), dim3(256), j0, j1);
    return launch_kernel(g, pack_kernel<uint16_t>, dim3(grid), dim3(256), j0, j1);
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
    const PackJob none = make_job(nullptr, 8, 0, 0, false, nullptr, 2);
    const PackJob ja = pl.a.in_place ? none : make_job(g.A, g.lda, g.M, g.K, g.ta, wa, 2);
    const PackJob jb = pl.b.in_place ? none : make_job(g.B, g.ldb, g.N, g.K, !g.tb, wb, 2);
    hipError_t e = launch_pack(g, ja, jb, 2);
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

// INT8 operands the direct kernel cannot read (a pointer off a 16-byte
// boundary, a leading dimension that is not a whole number of 16-byte chunks, K
// not a multiple of its 128-deep k-tile) are read by the register-staged INT8
// kernels a byte at a time: 1000^3 took 66.6 us against 11.4 us for 1024^3.
// Both operands are copied here as k-contiguous row images, A' (M x K') and B'
// (N x K', B transposed), K' = K rounded up to 128 and zero-filled (each extra
// term is an exact zero product, so the INT32 sums are those of the call), rows
// on 128-byte lines; the product of the copies then takes the configuration
// the selection gives aligned operands of that shape (i8_select).  (Aligned
// operands with K a multiple of 16 need no copy: the interleaved direct kernel
// takes a partial first k-tile.)  Either
// operand already k-contiguous, aligned, on whole lines and with K a multiple
// of 128 is read in place.
int64_t packed8_workspace_bytes(const GemmArgs& g) {
    const int64_t kp = round_up(g.K, 128);
    const bool kt = g.K % 128 == 0;
    const bool a_in = kt && !g.ta && aligned16(g.A) && g.lda % 128 == 0;
    const bool b_in = kt && g.tb && aligned16(g.B) && g.ldb % 128 == 0;
    const int64_t a = a_in ? 0 : round_up(g.M * kp, kWorkspaceAlign);
    const int64_t b = b_in ? 0 : g.N * kp;
    return a + b;
}

hipError_t launch_packed8(const GemmArgs& g) {
    const int64_t kp = round_up(g.K, 128);
    const bool kt = g.K % 128 == 0;
    const bool a_in = kt && !g.ta && aligned16(g.A) && g.lda % 128 == 0;
    const bool b_in = kt && g.tb && aligned16(g.B) && g.ldb % 128 == 0;
    if (a_in && b_in) return launch_mfma_i8(g, i8_select(g.M, g.N, g.K, true, true));
    const int64_t need = packed8_workspace_bytes(g);
    if (g.ws == nullptr || (reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign) != 0 ||
        g.ws_bytes < need) {
        const bool aligned = aligned16(g.A) && aligned16(g.B) && g.lda % 16 == 0 &&
                             g.ldb % 16 == 0;
        return launch_mfma_i8(g, i8_select(g.M, g.N, g.K, kt && aligned,
                                           g.K % 16 == 0 && aligned));
    }
    char* const wa = static_cast<char*>(g.ws);
    char* const wb = wa + (a_in ? 0 : round_up(g.M * kp, kWorkspaceAlign));
    const PackJob none = make_job(nullptr, 16, 0, 0, false, nullptr, 1);
    const PackJob ja = a_in ? none : make_job(g.A, g.lda, g.M, g.K, g.ta, wa, 1);
    const PackJob jb = b_in ? none : make_job(g.B, g.ldb, g.N, g.K, !g.tb, wb, 1);
    hipError_t e = launch_pack(g, ja, jb, 1);
    if (e != hipSuccess) return e;
    GemmArgs p = g;
    p.K = kp;
    if (!a_in) {
        p.ta = false;
        p.A = wa;
        p.lda = ja.ldd;
        p.pad_a = true;
    }
    if (!b_in) {
        p.tb = true;
        p.B = wb;
        p.ldb = jb.ldd;
        p.pad_b = true;
    }
    return launch_mfma_i8(p, i8_select(p.M, p.N, p.K, true, true));
}

// FP32 operands the direct kernel cannot read (a pointer off a 16-byte
// boundary, a leading dimension that is not a whole number of 4-element chunks,
// a contiguous side that ends inside a chunk) are read element by element by
// the register-staged FP32 kernels: 2049^3 took 399 us against 124 for 2048^3,
// 1023^3 45.3 against 20.4.  They are copied here like the 16-bit and 8-bit
// ones (4-byte elements, k-contiguous images with K zero-filled to a multiple
// of the 32-deep FP32 k-tile, rows on 128-byte lines), then the direct FP32
// kernel multiplies the copies: the 128x128 tile (configuration 10) from a
// round of its tiles, else the 64x64 one (8).  An operand the direct kernel
// reads in place (aligned, whole chunks, K a multiple of 4) is left in place.
namespace {

struct Plan32 {
    bool a_in, b_in;
    int64_t kp, a_bytes, b_bytes;
};

Plan32 plan32(const GemmArgs& g) {
    Plan32 p;
    const bool k4 = g.K % 4 == 0;
    p.kp = round_up(g.K, 32);
    p.a_in = k4 && aligned16(g.A) && g.lda % 4 == 0 && (!g.ta || g.M % 4 == 0);
    p.b_in = k4 && aligned16(g.B) && g.ldb % 4 == 0 && (g.tb || g.N % 4 == 0);
    p.a_bytes = p.a_in ? 0 : round_up(g.M * p.kp * 4, kWorkspaceAlign);
    p.b_bytes = p.b_in ? 0 : g.N * p.kp * 4;
    return p;
}

int inner32(const GemmArgs& g) { return f32_direct_tile(g.M, g.N); }

}  // namespace

int64_t packed32_workspace_bytes(const GemmArgs& g) {
    const Plan32 p = plan32(g);
    return p.a_bytes + p.b_bytes;
}

hipError_t launch_packed32(const GemmArgs& g) {
    const Plan32 pl = plan32(g);
    const int64_t need = pl.a_bytes + pl.b_bytes;
    if (need == 0) return launch_regtile_mfma(g, inner32(g));
    if (g.ws == nullptr || (reinterpret_cast<uintptr_t>(g.ws) % kWorkspaceAlign) != 0 ||
        g.ws_bytes < need)
        return launch_regtile_mfma(g, ceil_div(g.M, 128) * ceil_div(g.N, 128) >= 256 ? 0 : 2);
    char* const wa = static_cast<char*>(g.ws);
    char* const wb = wa + pl.a_bytes;
    const PackJob none = make_job(nullptr, 4, 0, 0, false, nullptr, 4);
    const PackJob ja = pl.a_in ? none : make_job(g.A, g.lda, g.M, g.K, g.ta, wa, 4);
    const PackJob jb = pl.b_in ? none : make_job(g.B, g.ldb, g.N, g.K, !g.tb, wb, 4);
    hipError_t e = launch_pack(g, ja, jb, 4);
    if (e != hipSuccess) return e;
    GemmArgs p = g;
    // Both operands copies: whole k-tiles of zero-filled K.  One left in place:
    // the call's K (the direct kernel zero-fills a partial last k-tile).
    if (!pl.a_in && !pl.b_in) p.K = pl.kp;
    if (!pl.a_in) {
        p.ta = false;
        p.A = wa;
        p.lda = ja.ldd;
        p.pad_a = true;
    }
    if (!pl.b_in) {
        p.tb = true;
        p.B = wb;
        p.ldb = jb.ldd;
        p.pad_b = true;
    }
    return launch_regtile_mfma(p, inner32(p));
}

}  // namespace migemm
