// common.hpp -- internal types shared by the kernels and the C ABI of the
// gfx950 GEMM library.  Not installed; the public interface is migemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace migemm {

// The output step of one product: where C lives and how the FP32 sum of
// products v of each element becomes that element.  Plain (alpha = 1, beta = 0,
// FP32 C): C = v.  General: C = alpha v + beta C_old, in FP32 (beta == 0 leaves
// C_old unread), then rounded to nearest even into the output format (page
// "CUDA-Practice 09", section on FP32 accumulation: the accumulator is written
// back as FP32 or rounded as required; page "matmul_registers.cu", the library
// call scaling the product by alpha and the previous C by beta).
struct Epi {
    void* C;
    int64_t ldc;
    float alpha, beta;
    int c_dtype;  // 0 FP32, 1 FP16, 2 BF16, 4 INT32 (INT8 products only; plain overwrite)
};

// The kernels one call would launch, recorded instead of launched when a
// GemmArgs carries a query (migemm_describe): host stubs for the HIP attribute
// queries, with each launch's workgroup count and size.
struct LaunchInfo {
    static constexpr int kMax = 4;
    int count = 0;
    const void* fn[kMax] = {};
    unsigned grid[kMax] = {}, block[kMax] = {};
    void add(const void* f, unsigned g, unsigned b) {
        if (count < kMax) {
            fn[count] = f;
            grid[count] = g;
            block[count] = b;
        }
        ++count;
    }
};

// Arguments of one product, already validated by the C ABI.  ta: A is given
// transposed, stored K x M (element (i, k) at A[k * lda + i]); tb: B is given
// transposed, stored N x K (element (k, j) at B[j * ldb + k]).  ws / ws_bytes:
// device workspace the caller lent to this call (packed operands), or none.
struct GemmArgs {
    int64_t M, N, K;
    int dtype;
    bool ta, tb;
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    Epi out;
    hipStream_t stream;
    void* ws = nullptr;
    int64_t ws_bytes = 0;
    LaunchInfo* query = nullptr;
    // The operand is a copy made by the packed path: its contiguous side (k of a
    // row-major A or of B given transposed, m or n of the others) is zero-filled
    // up to a whole 16-byte chunk inside its leading dimension, so a kernel may
    // read that last chunk whole.
    bool pad_a = false, pad_b = false;
    // Only for the skinny kernel: element (i, j) of this product is C[j * ldc +
    // i], i.e. the call computes a block of C^T (the last columns of a product,
    // as B^T A^T).
    bool trans_c = false;
    // Split-K (direct configurations with flag bit 7 only): the launch runs
    // `splitk` slices of K (splitk_slice), slice y writing its plain sums (FP32,
    // INT32 for 8-bit inputs) to the y-th M x N block of out.C.  0 or 1: one
    // ordinary launch.
    int splitk = 0;
    // True unless the output step is the plain FP32 overwrite.
    bool general() const { return !(out.alpha == 1.0f && out.beta == 0.0f && out.c_dtype == 0); }
};

// Launches fn<<<grid, block>>>(args...) on the call's stream, or, when the call
// is a query, records the launch instead.
template <typename... P, typename... Args>
hipError_t launch_kernel(const GemmArgs& g, void (*fn)(P...), dim3 grid, dim3 block,
                         Args&&... args) {
    if (g.query) {
        g.query->add(reinterpret_cast<const void*>(fn), grid.x * grid.y * grid.z,
                     block.x * block.y * block.z);
        return hipSuccess;
    }
    fn<<<grid, block, 0, g.stream>>>(std::forward<Args>(args)...);
    return hipGetLastError();
}

// Whether every row of C starts a 128-byte line (C aligned to a line, ldc a
// whole number of lines).  Non-temporal C stores pay only then: the row pieces
// that neighbouring 16x16 blocks store fill whole lines.  Rows that straddle
// lines (an odd ldc, say) split every piece into two partial-line writes, which
// plain stores merge in L2 and non-temporal ones send on as they are (the
// 2050 x 2047 FP16 product ran 18% slower with them, 4096^3 BF16 with ldc 4104
// 24%), so the direct configurations with non-temporal stores have plain-store
// twins for such C.
inline bool c_whole_lines(const Epi& o) {
    const int64_t eb = (o.c_dtype == 1 || o.c_dtype == 2) ? 2 : 4;
    return (o.ldc * eb) % 128 == 0 && (reinterpret_cast<uintptr_t>(o.C) & 127) == 0;
}

// Split-K: the k extent of each of `slices` slices of K, a whole number of
// `unit` (64, or the 128-deep INT8 k-tile) (the last slice takes what is left).
// With slices = ceil(K / splitk_slice(K, s, unit)) slices, every slice is
// non-empty and this gives the same extent again (checked for every K below
// 2^17 and s from 2 to 16).
__host__ __device__ inline int64_t splitk_slice(int64_t K, int64_t slices, int64_t unit = 64) {
    const int64_t c = (K + slices - 1) / slices;
    return (c + unit - 1) / unit * unit;
}

// Storage of a bfloat16 element: its 16 bits.
struct bf16_t {
    uint16_t bits;
};

// Element widening to FP32.  Every FP16 and BF16 value is exactly
// representable in FP32, so these are exact.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// FP32 -> BF16 bits, round to nearest even (gfx950 converts in hardware; NaN
// stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// The previous value of element idx of C, widened to FP32 (general form, beta != 0).
__device__ __forceinline__ float load_prev(const Epi& e, int64_t idx) {
    if (e.c_dtype == 0) return static_cast<const float*>(e.C)[idx];
    if (e.c_dtype == 1) return static_cast<float>(static_cast<const _Float16*>(e.C)[idx]);
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(e.C)[idx]) << 16);
}

// Stores alpha v + beta prev (alpha v when beta == 0), computed in FP32 and
// rounded to nearest even into the output format; NT selects non-temporal stores.
template <bool NT>
__device__ __forceinline__ void store_update(const Epi& e, int64_t idx, float v, float prev) {
    const float r = e.beta != 0.0f ? fmaf(e.alpha, v, e.beta * prev) : e.alpha * v;
    if (e.c_dtype == 4) {  // INT32 C: only the empty product (K == 0) comes here, with v == 0
        static_cast<int32_t*>(e.C)[idx] = static_cast<int32_t>(r);
    } else if (e.c_dtype == 0) {
        float* p = static_cast<float*>(e.C) + idx;
        if constexpr (NT)
            __builtin_nontemporal_store(r, p);
        else
            *p = r;
    } else if (e.c_dtype == 1) {
        _Float16* p = static_cast<_Float16*>(e.C) + idx;
        const _Float16 h = static_cast<_Float16>(r);
        if constexpr (NT)
            __builtin_nontemporal_store(h, p);
        else
            *p = h;
    } else {
        uint16_t* p = static_cast<uint16_t*>(e.C) + idx;
        const uint16_t b = f32_to_bf16_bits(r);
        if constexpr (NT)
            __builtin_nontemporal_store(b, p);
        else
            *p = b;
    }
}

// A streaming FP32 store: non-temporal, with device-wide coherence scope
// (sc1 nt).  When every workgroup finishes its tile at once, C leaves in one
// burst, and this policy measured about 1% faster on the 8192^3 product than the
// plain non-temporal store (`nt`).  A vector store like any other: only the cache
// policy bits differ.
__device__ __forceinline__ void store_f32_stream(float* p, float v) {
    asm volatile("global_store_dword %0, %1, off sc1 nt" : : "v"(p), "v"(v) : "memory");
}

// The same streaming store for INT32 C.
__device__ __forceinline__ void store_i32_stream(int32_t* p, int32_t v) {
    asm volatile("global_store_dword %0, %1, off sc1 nt" : : "v"(p), "v"(v) : "memory");
}

// Writes v, the FP32 sum of products of element idx (row * ldc + col) of C, as
// the output step says.  GEN == false is the plain FP32 overwrite (the only
// form the kernels compile for the default call); NT selects streaming
// stores.
template <bool GEN, bool NT = false>
__device__ __forceinline__ void store_out(const Epi& e, int64_t idx, float v) {
    if constexpr (!GEN) {
        float* p = static_cast<float*>(e.C) + idx;
        if constexpr (NT)
            store_f32_stream(p, v);
        else
            *p = v;
    } else {
        store_update<NT>(e, idx, v, e.beta != 0.0f ? load_prev(e, idx) : 0.0f);
    }
}

template <typename T> struct ZeroOf { static __device__ __forceinline__ T get() { return T(0); } };
template <> struct ZeroOf<bf16_t> {
    static __device__ __forceinline__ bf16_t get() { return bf16_t{0}; }
};

// 16-byte vector of raw bits (the unit of global and LDS traffic).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;  // gfx950 wavefront width
constexpr int kNumXcd = 8; // MI355X: 8 accelerator complex dies, 32 CUs each

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launchers, one per variant: return hipSuccess or the launch error.
// `config` is an index into that variant's configuration list.
hipError_t launch_naive(const GemmArgs& a, int config);
hipError_t launch_lds_tiled(const GemmArgs& a, int config);
hipError_t launch_regtile_valu(const GemmArgs& a, int config);
hipError_t launch_regtile_mfma(const GemmArgs& a, int config);
hipError_t launch_mfma16(const GemmArgs& a, int config);
// Packed configuration pc (11 or 12 of mfma16): packs the operands the direct
// kernel cannot read in place into zero-padded k-contiguous copies in the call's
// workspace and runs the configuration's direct kernel on them; runs
// fallback_config in place when the call lent no workspace of
// packed16_workspace_bytes(a, pc) bytes (pack.hip).
hipError_t launch_packed16(const GemmArgs& a, int pc, int fallback_config);
// Workspace bytes packed configuration pc needs for these arguments (0: both
// operands are read in place).
int64_t packed16_workspace_bytes(const GemmArgs& a, int pc);
// True when the call lent a workspace packed configuration pc can use:
// non-null, kWorkspaceAlign-aligned and at least packed16_workspace_bytes long.
bool packed16_workspace_ok(const GemmArgs& a, int pc);
// K rounded up to 64: the largest k extent of a packed copy.
int64_t packed_k(int64_t K);
// Alignment the packed path asks of a workspace.
constexpr int64_t kWorkspaceAlign = 256;
hipError_t launch_mfma_i8(const GemmArgs& a, int config);
// The INT8 configuration the selection gives this shape, with operands the
// direct kernels read with K a multiple of 128 (direct) or of 16 (direct16)
// (api.cpp).
int i8_select(int64_t M, int64_t N, int64_t K, bool direct, bool direct16);
// INT8 operands copied into aligned k-contiguous images, K zero-filled to a
// multiple of 128, in packed8_workspace_bytes(a) of the lent workspace, then
// the product of the copies (pack.hip; configuration 5 of the INT8 variant).
int64_t packed8_workspace_bytes(const GemmArgs& a);
hipError_t launch_packed8(const GemmArgs& a);
// The same for FP32 operands (configuration 13 of the FP32 matrix-core variant).
int64_t packed32_workspace_bytes(const GemmArgs& a);
hipError_t launch_packed32(const GemmArgs& a);
// FP16/BF16 products as slices of K on the 128x128 or 256x256 direct tile
// into FP32 partial sums in the caller's workspace, then a reduction that sums
// them in slice order and applies the output step (splitk.hip).
struct SplitKPlan {
    int config;      // the direct configuration that runs the slices: 7 or 10
    int64_t slices;  // 2 to 16 (1 where K holds a single whole k-tile slice)
};
// shallowest slices for the 256x256 tile: in general, and where the 128x128
// tile's slices would overshoot a round of 256 workgroups
constexpr int64_t kMinSlice256 = 4096, kMinSlice256Overshoot = 1024;
SplitKPlan splitk16_plan(const GemmArgs& g);
int64_t splitk16_slices(const GemmArgs& g);
int64_t splitk16_workspace_bytes(const GemmArgs& g);
hipError_t launch_splitk16(const GemmArgs& g);
// The same for FP32 operands: slices on the direct 64x64 FP32 tile
// (configuration 8 of the FP32 matrix-core variant), as many as make a round of
// 256 workgroups (2 to 16).
int64_t splitk32_slices(const GemmArgs& g);
int64_t splitk32_workspace_bytes(const GemmArgs& g);
hipError_t launch_splitk32(const GemmArgs& g);
// The same for INT8 operands: slices (whole 128-deep k-tiles) on the
// interleaved direct 256x256 INT8 tile (configuration 6), their exact INT32
// sums added by an integer sum kernel (configuration 7 of the INT8 variant).
int64_t splitk8_slices(const GemmArgs& g);
int64_t splitk8_workspace_bytes(const GemmArgs& g);
hipError_t launch_splitk8(const GemmArgs& g);
// FP32, FP16 and BF16 products with 1 <= M <= 16, K split over the waves of
// each workgroup (skinny.hip); skinny_fits says whether its alignment and
// whole-chunk needs hold (hipErrorInvalidValue from the launcher otherwise).
bool skinny_fits(const GemmArgs& a);
hipError_t launch_skinny(const GemmArgs& a);

// A tiled launch whose last band of tile rows or columns would start a round of
// workgroups of its own (split.cpp): the whole tiles first, then the rows past
// them, then the columns past them (rows [0, m_main) when the rows are split
// too), each tail of up to 16 on the skinny kernel (the columns as the
// transposed product), wider ones on a smaller tile.
struct SplitPlan {
    bool rows = false, cols = false;
    int64_t m_main = 0, n_main = 0;
};
// Tiles of bm x bn on the 256 CUs; tails wider than max_tail are not split off.
SplitPlan plan_split(int64_t M, int64_t N, int64_t bm, int64_t bn, int64_t max_tail);
// The direct FP32 tile for an M x N product: 10 (128x128) or 8 (64x64), whichever
// leaves fewer rounds of workgroups per CU (ties to the larger tile).
int f32_direct_tile(int64_t M, int64_t N);
using CfgLauncher = hipError_t (*)(const GemmArgs&, int);
hipError_t launch_split(const GemmArgs& g, const SplitPlan& p, CfgLauncher head, int head_config,
                        CfgLauncher tail, int tail_config);
// K == 0: the sum of products is 0 for every element; applies the output step to it.
hipError_t launch_empty_product(const GemmArgs& a);

// dst (rows x cols, ldd, dst_dtype) = src (rows x cols, lds, src_dtype) converted,
// round to nearest even where narrower.
hipError_t launch_convert(int src_dtype, int dst_dtype, int64_t rows, int64_t cols,
                          const void* src, int64_t lds, void* dst, int64_t ldd, hipStream_t s);

// The C ABI's common path (api.cpp): validates one call, selects its variant
// and configuration (variant -1: the selection table's; config -1: the table's
// choice for the variant), and launches it with the workspace lent (ws may be
// NULL).  Returns a migemm_status.
int run_gemm(int variant, int config, int op_a, int op_b, int64_t M, int64_t N, int64_t K,
             int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, float alpha,
             float beta, int c_dtype, void* C, int64_t ldc, void* ws, int64_t ws_bytes,
             void* stream);
// The workspace bytes such a call uses when lent enough (api.cpp).
int workspace_bytes(int variant, int config, int op_a, int op_b, int64_t M, int64_t N,
                    int64_t K, int dtype, const void* A, int64_t lda, const void* B,
                    int64_t ldb, int64_t* bytes);

// Configuration tables, one per variant (names, and the count).
int naive_config_count();
const char* naive_config_name(int c);
int lds_tiled_config_count();
const char* lds_tiled_config_name(int c);
int regtile_valu_config_count();
const char* regtile_valu_config_name(int c);
int regtile_mfma_config_count();
const char* regtile_mfma_config_name(int c);
int mfma16_config_count();
const char* mfma16_config_name(int c);
int mfma_i8_config_count();
const char* mfma_i8_config_name(int c);

}  // namespace migemm
