// api.cpp -- the C ABI (migemm.h): argument checks, the variant registry,
// the deterministic selection table, and stream-ordered launch.
//
// The library's interface is a status-returning call in the manner of the
// vendor GEMM call on page "matmul_registers.cu" (section on the library
// comparison, where the status goes back to the caller rather than aborting):
// nothing here prints, throws or exits.  The one allocation is the workspace of
// the packed FP16/BF16 configurations (pack.hip): a buffer per device, allocated
// on first use and kept; a call that needs a larger one waits for the previous
// user of the buffer before reallocating it, the only host-side wait.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "migemm.h"

namespace migemm {
namespace {

// Sizes are limited so that every index product fits in 64 bits:
// a dimension below 2^31 times a leading dimension below 2^32.
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxLd = int64_t(1) << 32;
// M * N * K from which a 16-bit product the direct kernel cannot read in place
// is run on packed copies (pack.hip) rather than by the register-staged kernel.
constexpr double kPackMinWork = 134217728.0;  // 2^27, e.g. 512^3

struct Variant {
    const char* name;
    unsigned dtype_mask;  // bit d set: takes dtype d
    int (*count)();
    const char* (*config_name)(int);
    hipError_t (*launch)(const GemmArgs&, int);
};

const Variant kVariants[] = {
    {"naive", 0x7u, naive_config_count, naive_config_name, launch_naive},
    {"lds_tiled", 0x1u, lds_tiled_config_count, lds_tiled_config_name, launch_lds_tiled},
    {"regtile_valu", 0x1u, regtile_valu_config_count, regtile_valu_config_name,
     launch_regtile_valu},
    {"regtile_mfma", 0x1u, regtile_mfma_config_count, regtile_mfma_config_name,
     launch_regtile_mfma},
    {"mfma16", 0x6u, mfma16_config_count, mfma16_config_name, launch_mfma16},
    {"mfma_i8", 0x8u, mfma_i8_config_count, mfma_i8_config_name, launch_mfma_i8},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

thread_local int g_last_hip_error = 0;

int elem_size(int dtype) {
    return (dtype == MIGEMM_F32 || dtype == MIGEMM_I32) ? 4 : dtype == MIGEMM_I8 ? 1 : 2;
}

// INT8: each product is at most 2^14 in magnitude ((-128)(-128)), so sums of at
// most 2^17 - 1 of them stay below 2^31 and fit INT32 exactly.
constexpr int64_t kMaxKi8 = (int64_t(1) << 17) - 1;

// Byte range [lo, hi) touched by a rows x cols row-major operand with leading dimension ld.
void extent(const void* p, int64_t rows, int64_t cols, int64_t ld, int es, uintptr_t& lo,
            uintptr_t& hi) {
    lo = reinterpret_cast<uintptr_t>(p);
    hi = lo + static_cast<uintptr_t>(((rows - 1) * ld + cols) * es);
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

bool known_dtype(int d) { return d == MIGEMM_F32 || d == MIGEMM_F16 || d == MIGEMM_BF16; }
bool known_input(int d) { return known_dtype(d) || d == MIGEMM_I8; }
bool known_output(int d) { return known_dtype(d) || d == MIGEMM_I32; }

bool known_op(int op) { return op == MIGEMM_OP_N || op == MIGEMM_OP_T; }

// ta / tb: the operand is given transposed, so its stored rows run along k (A,
// stored K x M) or along n (B, stored N x K).
int check_args(int64_t M, int64_t N, int64_t K, int dtype, bool ta, bool tb, const void* A,
               int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc, int c_dtype,
               bool need_ptrs) {
    if (!known_input(dtype) || !known_output(c_dtype)) return MIGEMM_ERR_INVALID_ARG;
    // INT8 inputs go with INT32 C and nothing else does
    if ((dtype == MIGEMM_I8) != (c_dtype == MIGEMM_I32)) return MIGEMM_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return MIGEMM_ERR_INVALID_ARG;
    if (dtype == MIGEMM_I8 && K > kMaxKi8) return MIGEMM_ERR_INVALID_ARG;
    auto at_least = [](int64_t ld, int64_t cols) { return ld >= (cols > 1 ? cols : 1); };
    if (!at_least(lda, ta ? M : K) || !at_least(ldb, tb ? K : N) || !at_least(ldc, N))
        return MIGEMM_ERR_INVALID_ARG;
    if (lda > kMaxLd || ldb > kMaxLd || ldc > kMaxLd) return MIGEMM_ERR_INVALID_ARG;
    if (!need_ptrs) return MIGEMM_OK;
    if ((M > 0 && K > 0 && !A) || (K > 0 && N > 0 && !B) || (M > 0 && N > 0 && !C))
        return MIGEMM_ERR_INVALID_ARG;
    if (M > 0 && N > 0) {
        const int es = elem_size(dtype);
        uintptr_t c0, c1;
        extent(C, M, N, ldc, elem_size(c_dtype), c0, c1);
        if (K > 0) {
            uintptr_t a0, a1, b0, b1;
            if (ta)
                extent(A, K, M, lda, es, a0, a1);
            else
                extent(A, M, K, lda, es, a0, a1);
            if (tb)
                extent(B, N, K, ldb, es, b0, b1);
            else
                extent(B, K, N, ldb, es, b0, b1);
            if (overlaps(c0, c1, a0, a1) || overlaps(c0, c1, b0, b1)) return MIGEMM_ERR_INVALID_ARG;
        }
    }
    return MIGEMM_OK;
}

// 16-byte aligned operand pointers with leading dimensions of whole 16-byte
// chunks (8 16-bit or 16 8-bit elements).  NULL pointers count as aligned
// (migemm_select).
bool operands_aligned(const void* A, int64_t lda, const void* B, int64_t ldb, int dtype) {
    const int64_t epc = dtype == MIGEMM_I8 ? 16 : 8;
    return aligned16(A) && aligned16(B) && lda % epc == 0 && ldb % epc == 0;
}

// The selection table: a pure function of shape, dtype, operand layout and
// alignment.  Sizes are bucketed by how many workgroup tiles a configuration
// would launch against the 256 CUs of an MI355X.
void select(int64_t M, int64_t N, int64_t K, int dtype, bool ta, bool tb, bool aligned,
            int& variant, int& config) {
    auto tiles = [&](int64_t bm, int64_t bn) { return ceil_div(M, bm) * ceil_div(N, bn); };
    if (dtype == MIGEMM_I8) {
        variant = MIGEMM_MFMA_I8;
        // whole 256x256 tiles with aligned operands: the direct ping-pong kernel;
        // otherwise the register-staged 256x256 with 32x32x32 instructions
        // measured best in every layout at 8192^3
        const bool whole = M % 256 == 0 && N % 256 == 0 && K % 128 == 0 && aligned;
        config = tiles(256, 256) >= 256 ? (whole ? 4 : 3) : tiles(128, 128) >= 256 ? 1 : 2;
        return;
    }
    if (dtype == MIGEMM_F32) {
        variant = MIGEMM_REGTILE_MFMA;
        config = tiles(128, 128) >= 256 ? 0 : 2;
        return;
    }
    variant = MIGEMM_MFMA16;
    // Direct global->LDS staging needs 16-byte aligned operands with leading
    // dimensions a multiple of 8 elements, K a multiple of 64, and N (row-major
    // B) or M (A given transposed) a multiple of 8; the launcher falls back to
    // the register-staged kernel otherwise.  Other operands are packed into
    // zero-padded copies for the direct kernel once the product is large
    // enough for the two extra copy launches to pay.
    const bool direct = aligned && K % 64 == 0 && (tb || N % 8 == 0) && (!ta || M % 8 == 0);
    const double work = static_cast<double>(M) * static_cast<double>(N) * static_cast<double>(K);
    const bool pack = work >= kPackMinWork && packed_k(K) < (int64_t(1) << 21);
    const bool whole256 = M % 256 == 0 && N % 256 == 0;
    if (direct && tiles(256, 256) >= 256 && whole256)
        config = 14;  // direct 256x256x64, ping-pong wave groups (whole tiles only)
    else if (direct && tiles(256, 256) >= 256)
        config = 10;  // direct 256x256x64, 8 waves, 16x16x32, AGPR accumulators, early loads
    else if (direct && tiles(128, 256) >= 256 && M % 128 == 0 && N % 256 == 0)
        config = 15;  // direct 128x256x64, ping-pong wave groups (e.g. 1024x8192, 4096x2048)
    else if (direct && tiles(128, 256) >= 256)
        config = 13;  // direct 128x256x64, 8 waves of 64x64, 3 stages
    else if (direct && tiles(128, 128) >= 256)
        config = 7;   // direct 128x128x64, 8 waves, 4 stages, interleaved
    else if (direct)
        config = 16;  // direct 64x64x64, 8 waves: four times the workgroups (e.g. 1024^3)
    else if (pack)
        config = tiles(256, 256) >= 256 ? 11 : 12;  // packed copies, then config 14/10 or 7
    else if (tiles(128, 128) >= 256)
        config = 2;   // register-staged 128x128x64
    else
        config = 3;   // register-staged 64x64x64
}

int run(int variant, int config, int op_a, int op_b, int64_t M, int64_t N, int64_t K,
        int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, float alpha,
        float beta, int c_dtype, void* C, int64_t ldc, void* stream) {
    if (!known_op(op_a) || !known_op(op_b)) return MIGEMM_ERR_INVALID_ARG;
    const bool ta = op_a == MIGEMM_OP_T, tb = op_b == MIGEMM_OP_T;
    int st = check_args(M, N, K, dtype, ta, tb, A, lda, B, ldb, C, ldc, c_dtype, true);
    if (st != MIGEMM_OK) return st;
    // INT32 C takes the plain product only
    if (c_dtype == MIGEMM_I32 && (alpha != 1.0f || beta != 0.0f)) return MIGEMM_ERR_UNSUPPORTED;
    const bool aligned = operands_aligned(A, lda, B, ldb, dtype);
    if (variant == MIGEMM_VARIANT_AUTO) {
        if (config != -1) return MIGEMM_ERR_INVALID_ARG;
        select(M, N, K, dtype, ta, tb, aligned, variant, config);
    }
    if (variant < 0 || variant >= kNumVariants) return MIGEMM_ERR_INVALID_ARG;
    const Variant& v = kVariants[variant];
    if (!(v.dtype_mask & (1u << dtype))) return MIGEMM_ERR_UNSUPPORTED;
    if (config == -1) {
        int sv, sc;
        select(M, N, K, dtype, ta, tb, aligned, sv, sc);
        config = (sv == variant) ? sc : 0;
    }
    if (config < 0 || config >= v.count()) return MIGEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return MIGEMM_OK;

    const GemmArgs g{M,   N,   K, dtype, ta, tb, A, lda, B, ldb,
                     Epi{C, ldc, alpha, beta, c_dtype}, static_cast<hipStream_t>(stream)};
    const hipError_t err = K == 0 ? launch_empty_product(g) : v.launch(g, config);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return MIGEMM_ERR_HIP;
    }
    return MIGEMM_OK;
}

}  // namespace
}  // namespace migemm

using namespace migemm;

extern "C" {

int migemm_gemm(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                const void* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
    return run(MIGEMM_VARIANT_AUTO, -1, MIGEMM_OP_N, MIGEMM_OP_N, M, N, K, dtype, A, lda, B, ldb,
               1.0f, 0.0f, MIGEMM_F32, C, ldc, stream);
}

int migemm_gemm_variant(int variant, int config, int64_t M, int64_t N, int64_t K, int dtype,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                        int64_t ldc, void* stream) {
    return run(variant, config, MIGEMM_OP_N, MIGEMM_OP_N, M, N, K, dtype, A, lda, B, ldb, 1.0f,
               0.0f, MIGEMM_F32, C, ldc, stream);
}

int migemm_gemm_ex(int op_a, int op_b, int64_t M, int64_t N, int64_t K, int dtype, const void* A,
                   int64_t lda, const void* B, int64_t ldb, float alpha, float beta, int c_dtype,
                   void* C, int64_t ldc, void* stream) {
    return run(MIGEMM_VARIANT_AUTO, -1, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha, beta,
               c_dtype, C, ldc, stream);
}

int migemm_gemm_ex_variant(int variant, int config, int op_a, int op_b, int64_t M, int64_t N,
                           int64_t K, int dtype, const void* A, int64_t lda, const void* B,
                           int64_t ldb, float alpha, float beta, int c_dtype, void* C,
                           int64_t ldc, void* stream) {
    return run(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha, beta, c_dtype,
               C, ldc, stream);
}

int migemm_convert(int src_dtype, int dst_dtype, int64_t rows, int64_t cols, const void* src,
                   int64_t lds, void* dst, int64_t ldd, void* stream) {
    if (!known_dtype(src_dtype) || !known_dtype(dst_dtype)) return MIGEMM_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return MIGEMM_ERR_INVALID_ARG;
    const int64_t min_ld = cols > 1 ? cols : 1;
    if (lds < min_ld || ldd < min_ld || lds > kMaxLd || ldd > kMaxLd) return MIGEMM_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return MIGEMM_OK;
    if (!src || !dst) return MIGEMM_ERR_INVALID_ARG;
    uintptr_t s0, s1, d0, d1;
    extent(src, rows, cols, lds, elem_size(src_dtype), s0, s1);
    extent(dst, rows, cols, ldd, elem_size(dst_dtype), d0, d1);
    if (overlaps(s0, s1, d0, d1)) return MIGEMM_ERR_INVALID_ARG;
    const hipError_t err = launch_convert(src_dtype, dst_dtype, rows, cols, src, lds, dst, ldd,
                                          static_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return MIGEMM_ERR_HIP;
    }
    return MIGEMM_OK;
}

int migemm_variant_count(void) { return kNumVariants; }

const char* migemm_variant_name(int variant) {
    return (variant >= 0 && variant < kNumVariants) ? kVariants[variant].name : nullptr;
}

int migemm_variant_supports(int variant, int dtype) {
    if (variant < 0 || variant >= kNumVariants || !known_input(dtype)) return 0;
    return (kVariants[variant].dtype_mask >> dtype) & 1u;
}

int migemm_config_count(int variant) {
    return (variant >= 0 && variant < kNumVariants) ? kVariants[variant].count() : 0;
}

const char* migemm_config_name(int variant, int config) {
    if (variant < 0 || variant >= kNumVariants) return nullptr;
    return kVariants[variant].config_name(config);
}

int migemm_select(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                  const void* B, int64_t ldb, const float* C, int64_t ldc, int* variant,
                  int* config) {
    (void)A;
    (void)B;
    (void)C;
    const int c_dtype = dtype == MIGEMM_I8 ? MIGEMM_I32 : MIGEMM_F32;
    int st = check_args(M, N, K, dtype, false, false, A, lda, B, ldb, C, ldc, c_dtype, false);
    if (st != MIGEMM_OK) return st;
    if (!variant || !config) return MIGEMM_ERR_INVALID_ARG;
    select(M, N, K, dtype, false, false, operands_aligned(A, lda, B, ldb, dtype), *variant, *config);
    return MIGEMM_OK;
}

const char* migemm_status_string(int status) {
    switch (status) {
        case MIGEMM_OK: return "ok";
        case MIGEMM_ERR_INVALID_ARG: return "invalid argument";
        case MIGEMM_ERR_UNSUPPORTED: return "variant does not support this dtype";
        case MIGEMM_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int migemm_last_hip_error(void) { return g_last_hip_error; }

int migemm_version(void) { return 500; }

}  // extern "C"
