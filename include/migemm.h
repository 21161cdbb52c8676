/*
 * migemm.h -- C ABI of the MI355X (gfx950) dense matrix-multiply library.
 *
 * Operation.  C = A x B, overwriting C, for row-major A (M x K), B (K x N) and
 * C (M x N):
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 *
 * (page "Tensor cores and matrix operations", section "Traditional Approach:
 * Element-by-Element"; the product is a plain overwrite, alpha = 1 and
 * beta = 0, as in the library call on page "matmul_registers.cu").  Two forms:
 *
 *   MIGEMM_F32   FP32 A and B, FP32 arithmetic, FP32 C (the FP32 GEMMs of
 *                pages "matmul_registers.cu" and "04-wmma-matmul.cu");
 *   MIGEMM_F16,  FP16 or BF16 A and B, products accumulated in FP32, FP32 C
 *   MIGEMM_BF16  (page "CUDA-Practice 09", section on mixed precision: half
 *                inputs halve the bytes read, FP32 accumulation keeps long sums
 *                from losing small terms).
 *
 * Layout.  Row-major with leading dimensions in ELEMENTS: element (i, k) of A
 * is at A[i * lda + k], (k, j) of B at B[k * ldb + j], (i, j) of C at
 * C[i * ldc + j].  Requirements: lda >= max(1, K), ldb >= max(1, N),
 * ldc >= max(1, N), each leading dimension below 2^32 and M, N, K below 2^31
 * (so every index product fits in 64 bits), and every operand's byte range
 * inside the address space.  No alignment is required; 16-byte aligned pointers and
 * leading dimensions that are multiples of 16 bytes take the vector-load path.
 *
 * Pointers.  A, B and C are DEVICE pointers on the current HIP device, owned
 * by the caller.  The library keeps no pointer of the caller's after a call
 * returns.  Calls are reentrant and may come from several host threads.  C
 * must not overlap A or B.
 *
 * Memory.  The library allocates no device memory.  FP16/BF16 operands that
 * the direct-staged kernel cannot read in place (rows not 16-byte aligned in
 * whole 16-byte chunks, K or a k-row image side not a multiple of 8) or reads
 * slowly (k-contiguous rows that do not start on 128-byte lines) are, for
 * large products, best first copied into zero-padded k-contiguous images (so
 * are INT8 operands the direct kernels cannot read); and products whose M x N
 * is a few tiles beside a long K are best summed as slices of K whose sums are
 * then added.  Both paths need device scratch memory, which the caller lends to
 * migemm_gemm_ws (its size from migemm_workspace_size).  The other entry points
 * lend none, and such products then run in place: same result rules, lower
 * speed.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Work is enqueued asynchronously on it; no entry point waits on the
 * host.  The caller synchronises before reading C.
 *
 * Errors.  Every entry point returns a migemm_status; nothing prints, throws
 * or exits.  Argument errors are detected before any HIP call.  Degenerate
 * shapes: M == 0 or N == 0 is a no-op returning MIGEMM_OK; K == 0 writes
 * C = 0 (an empty sum) over the M x N window.
 *
 * The general form migemm_gemm_ex adds the scaled update C = alpha A B + beta C
 * and FP16/BF16 storage of C (below).
 */
#ifndef MIGEMM_H
#define MIGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of A and B (and of C for migemm_gemm_ex; migemm_gemm's C is FP32). */
typedef enum {
    MIGEMM_F32 = 0,
    MIGEMM_F16 = 1,  /* IEEE binary16 */
    MIGEMM_BF16 = 2, /* bfloat16: the upper half of a binary32 word */
    MIGEMM_I8 = 3,   /* 8-bit two's-complement integer (inputs of migemm_gemm_ex only) */
    MIGEMM_I32 = 4   /* 32-bit integer (C of an INT8 product only) */
} migemm_dtype;

/*
 * Operand layout for migemm_gemm_ex (page "Tensor cores and matrix operations":
 * matrix-unit operands declared row-major or column-major; page
 * "matmul_registers.cu", library comparison: row-major operands handed to a
 * column-major library by swapping them).
 * MIGEMM_OP_N: the operand as stored is the one multiplied (A: M x K, element
 * (i, k) at A[i * lda + k]; B: K x N, element (k, j) at B[k * ldb + j]).
 * MIGEMM_OP_T: the operand is given transposed (A stored K x M: element (i, k)
 * at A[k * lda + i], lda >= max(1, M); B stored N x K: element (k, j) at
 * B[j * ldb + k], ldb >= max(1, K)).  A column-major operand is the transpose of
 * a row-major one with the same leading dimension, so OP_T also takes
 * column-major A or B.
 */
typedef enum { MIGEMM_OP_N = 0, MIGEMM_OP_T = 1 } migemm_op;

typedef enum {
    MIGEMM_OK = 0,
    MIGEMM_ERR_INVALID_ARG = 1, /* negative size, ld too small, unknown dtype, NULL with data,
                                   size beyond the supported range, bad variant/config index */
    MIGEMM_ERR_UNSUPPORTED = 2, /* a forced variant that does not take this dtype */
    MIGEMM_ERR_HIP = 3,         /* the HIP runtime reported an error at launch
                                   (see migemm_last_hip_error) */
    MIGEMM_ERR_WORKSPACE = 4    /* the product needs more scratch memory than the
                                   allocation-free entry point holds */
} migemm_status;

/*
 * Kernel variants.  Each one computes the same product; they differ in how
 * (and so in speed and in summation order, not in the tolerance they meet).
 *
 *   MIGEMM_NAIVE         one work-item per C element, FP32 fused multiply-adds
 *                        over k (page "04-wmma-matmul.cu", naiveMatmul; page
 *                        "CUDA-Practice 09", gemm_fp32_kernel).  All dtypes.
 *   MIGEMM_LDS_TILED     square tiles of A and B staged in LDS, one output per
 *                        work-item (page "matmul_registers.cu",
 *                        matmulSharedTiled).  FP32 only.
 *   MIGEMM_REGTILE_VALU  register micro-tiles per work-item with 16-byte global
 *                        loads and the A tile stored k-major in LDS (page
 *                        "matmul_registers.cu", matmulRegTile2d and
 *                        matmulRegTile2dVec4), on VALU FMA.  FP32 only.
 *   MIGEMM_REGTILE_MFMA  the same staging with the inner product on FP32
 *                        matrix-core instructions.  FP32 only.
 *   MIGEMM_MFMA16        FP16/BF16 matrix-core kernel with FP32 accumulation:
 *                        double-buffered, swizzled LDS tiles, 16-byte
 *                        coalesced staging (the tiled matrix-unit algorithm of
 *                        page "Tensor cores and matrix operations", section
 *                        "Complete Algorithm for Large Matrix Multiply").
 *                        FP16 and BF16 only.
 *   MIGEMM_MFMA_I8       the same algorithm on INT8 operands with exact INT32
 *                        sums (integer matrix-core instructions).  INT8 only.
 */
typedef enum {
    MIGEMM_VARIANT_AUTO = -1,
    MIGEMM_NAIVE = 0,
    MIGEMM_LDS_TILED = 1,
    MIGEMM_REGTILE_VALU = 2,
    MIGEMM_REGTILE_MFMA = 3,
    MIGEMM_MFMA16 = 4,
    MIGEMM_MFMA_I8 = 5
} migemm_variant;

/*
 * C = A x B with the variant and tile configuration chosen by the library's
 * selection table (deterministic: a pure function of the arguments).
 */
int migemm_gemm(int64_t M, int64_t N, int64_t K, int dtype,
                const void* A, int64_t lda, const void* B, int64_t ldb,
                float* C, int64_t ldc, void* stream);

/*
 * As migemm_gemm, with the variant forced (MIGEMM_VARIANT_AUTO selects as
 * migemm_gemm does) and the tile configuration forced by index
 * (config = -1: the selection table's choice for that variant).
 * MIGEMM_ERR_UNSUPPORTED if the variant does not take `dtype`;
 * MIGEMM_ERR_INVALID_ARG for an unknown variant or config index.
 */
int migemm_gemm_variant(int variant, int config,
                        int64_t M, int64_t N, int64_t K, int dtype,
                        const void* A, int64_t lda, const void* B, int64_t ldb,
                        float* C, int64_t ldc, void* stream);

/*
 * The general product:
 *
 *     C[i][j] = alpha * (sum_{k=0}^{K-1} A[i][k] * B[k][j]) + beta * C[i][j]
 *
 * the scaled update of the library call on page "matmul_registers.cu" (its
 * alpha multiplies the product, its beta the previous C), with C stored as FP32
 * or rounded into FP16 or BF16 (page "CUDA-Practice 09", section on FP32
 * accumulation: the FP32 accumulator is written back as FP32 or rounded as
 * required), and A and B each as stored or given transposed (op_a, op_b, see
 * migemm_op).
 *
 * The sum of products is the same FP32 accumulation, by the same kernels, as
 * migemm_gemm.  Per element the update is then computed in FP32 (beta * C_old
 * first, fused with alpha * sum) and rounded to nearest even into c_dtype
 * (MIGEMM_F32, MIGEMM_F16 or MIGEMM_BF16; magnitudes beyond the format's range
 * become +-infinity).  When beta == 0 the previous C is not read and may hold
 * anything, NaN included.  C points to c_dtype elements, row-major with leading
 * dimension ldc (elements).  K == 0 gives C = beta * C_old (or 0).
 * Same pointer, stream, ownership and error rules as migemm_gemm; an unknown
 * c_dtype or op is MIGEMM_ERR_INVALID_ARG, and C must not overlap A or B.
 *
 * INT8 (the integer variant of the matrix-unit product; the pages reach it only
 * through a link): dtype == MIGEMM_I8 takes c_dtype == MIGEMM_I32 and no other
 * (and MIGEMM_I32 only goes with MIGEMM_I8): C = A B exactly, in 32-bit two's
 * complement.  K is limited to 2^17 - 1, where no sum can overflow (each product
 * is at most 2^14 in magnitude); larger K is MIGEMM_ERR_INVALID_ARG.  Only the plain
 * product: alpha != 1 or beta != 0 is MIGEMM_ERR_UNSUPPORTED.
 * The selection depends on A, B, their layouts and the sizes only.
 * op_a == op_b == MIGEMM_OP_N with alpha == 1, beta == 0 and FP32 C is exactly
 * migemm_gemm.
 */
int migemm_gemm_ex(int op_a, int op_b, int64_t M, int64_t N, int64_t K, int dtype,
                   const void* A, int64_t lda, const void* B, int64_t ldb,
                   float alpha, float beta, int c_dtype, void* C, int64_t ldc,
                   void* stream);

/* As migemm_gemm_ex, with the variant and configuration forced as in
 * migemm_gemm_variant. */
int migemm_gemm_ex_variant(int variant, int config, int op_a, int op_b,
                           int64_t M, int64_t N, int64_t K, int dtype,
                           const void* A, int64_t lda, const void* B, int64_t ldb,
                           float alpha, float beta, int c_dtype, void* C, int64_t ldc,
                           void* stream);

/*
 * The most general product: migemm_gemm_ex_variant (variant and config forced,
 * or -1 for the selection table's choice) with device scratch memory lent by
 * the caller for this one call.
 *
 * workspace: NULL or a device pointer on the current device, 256-byte aligned,
 * of workspace_bytes bytes (>= 0), owned by the caller; the call's kernels
 * write it in stream order on `stream`, and the caller must not use it for
 * anything else until the work enqueued by this call has finished (stream
 * order on `stream` guarantees that for later work on the same stream).  The
 * library keeps no pointer to it after the call returns.  With at least the
 * size migemm_workspace_size reports for the same arguments, FP16/BF16
 * operands the direct-staged kernel cannot read in place are copied into
 * zero-padded k-contiguous images there (the padding adds only exact zero
 * terms to each sum, page "CUDA-Practice 09", the definition of the
 * row-major product), INT8 operands off 16-byte boundaries or with K not a
 * multiple of 16 likewise, FP32 ones off 16-byte boundaries or with K not a
 * multiple of 4 (M x N x K at least 2^27) likewise, and products of few tiles with a long K (FP16/BF16:
 * fewer than 256 tiles of 128 x 128, K at least 6144 and 4 max(M, N); FP32: at
 * most 128 tiles of 64 x 64, K at least 512; INT8: at most 64 tiles of
 * 256 x 256, K at least 8192) keep there the FP32 (INT32) sums of 2 to 16
 * slices of K (slices x M x N x 4 bytes), which a second kernel adds in slice
 * order, so the result does not depend on timing; a smaller, misaligned or
 * NULL workspace is not used and
 * the call runs a configuration that needs none.  The selection depends on
 * whether a usable workspace was lent.  Negative workspace_bytes is
 * MIGEMM_ERR_INVALID_ARG; otherwise the rules of migemm_gemm_ex apply.
 */
int migemm_gemm_ws(int variant, int config, int op_a, int op_b,
                   int64_t M, int64_t N, int64_t K, int dtype,
                   const void* A, int64_t lda, const void* B, int64_t ldb,
                   float alpha, float beta, int c_dtype, void* C, int64_t ldc,
                   void* workspace, int64_t workspace_bytes, void* stream);

/*
 * migemm_gemm_ws without a workspace argument, for callers that cannot
 * allocate device memory or lend a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  The scratch memory
 * comes from a fixed array of 64 MiB that the library's code object holds on
 * every GPU it runs on, from the time the library is first used there until the
 * process ends; the call itself allocates nothing.  A product that needs more
 * scratch than that (migemm_workspace_size reports more than 64 MiB) is
 * rejected with MIGEMM_ERR_WORKSPACE before any launch; products that need none
 * run at any size.  All calls on one GPU share its array, and each call's
 * kernels overwrite what they read of it, so nothing carries over between calls;
 * but calls whose work overlaps in time on one GPU (on different streams, or
 * from different host threads) race on the array: the caller orders them.
 * Otherwise exactly migemm_gemm_ws, with the same selection as a call lent a
 * 64 MiB workspace.
 */
int migemm_gemm_noalloc(int variant, int config, int op_a, int op_b,
                        int64_t M, int64_t N, int64_t K, int dtype,
                        const void* A, int64_t lda, const void* B, int64_t ldb,
                        float alpha, float beta, int c_dtype, void* C, int64_t ldc,
                        void* stream);

/*
 * Writes to *bytes the workspace migemm_gemm_ws uses for these arguments when
 * lent at least that much (0: none; the selection that lent workspace leads
 * to).  Pointers are only inspected for alignment and may be NULL (read as
 * 16-byte aligned).  Same argument checks as migemm_gemm_ex, and NULL `bytes`
 * is MIGEMM_ERR_INVALID_ARG.
 */
int migemm_workspace_size(int variant, int config, int op_a, int op_b,
                          int64_t M, int64_t N, int64_t K, int dtype,
                          const void* A, int64_t lda, const void* B, int64_t ldb,
                          int64_t* bytes);

/*
 * A description of what migemm_gemm would run for these sizes with 16-byte
 * aligned operands, for reports: the selected variant and configuration, the
 * workspace it would use, and for each kernel launch its workgroup count and
 * size and, where a GPU is present, the kernel's name, registers
 * (hipFuncGetAttributes numRegs), LDS and scratch bytes per workgroup and
 * workgroups per CU (occupancy).  The text is `key=value` pairs separated by
 * ';' (keys: variant, config, config_name, workspace_bytes, workspace_lent,
 * launches, then per launch i: grid<i>, block<i>, kernel<i>, regs<i>,
 * lds_bytes<i>, scratch_bytes<i>, max_block<i>, workgroups_per_cu<i>,
 * waves_per_simd<i>, or resources<i> when the attributes cannot be read).
 * Nothing is launched.  buf receives at most buflen - 1 characters and a
 * terminating NUL; MIGEMM_ERR_INVALID_ARG when buf is NULL, buflen < 1, the
 * text was cut short, or the arguments fail migemm_gemm's checks.
 */
int migemm_describe(int64_t M, int64_t N, int64_t K, int dtype,
                    int64_t lda, int64_t ldb, int64_t ldc, char* buf, int buflen);

/*
 * As migemm_describe, for the general call migemm_gemm_ws would make with
 * these arguments (variant and config forced or -1, operand layouts, operand
 * pointers inspected for alignment only, NULL read as 16-byte aligned, the
 * output type, and the workspace size that would be lent).
 */
int migemm_describe_ex(int variant, int config, int op_a, int op_b,
                       int64_t M, int64_t N, int64_t K, int dtype,
                       const void* A, int64_t lda, const void* B, int64_t ldb,
                       int c_dtype, int64_t ldc, int64_t workspace_bytes,
                       char* buf, int buflen);

/*
 * Element-type conversion of a matrix on the device, the step before the
 * product for FP32 data headed for the 16-bit matrix-core path (page
 * "04-wmma-matmul.cu": its FP32 inputs are converted to half before the
 * product; page "CUDA-Practice 09", section on mixed precision: 16-bit inputs
 * halve the bytes read):
 *
 *     dst[i][j] = src[i][j],  i < rows, j < cols
 *
 * from src_dtype to dst_dtype (any of MIGEMM_F32, MIGEMM_F16, MIGEMM_BF16).
 * Widening is exact; narrowing rounds to nearest even (magnitudes beyond the
 * target's range become +-infinity, NaN stays NaN).  Both matrices are
 * row-major device arrays with leading dimensions max(1, cols) <= lds, ldd < 2^32
 * (elements); elements between rows are not touched.  src and dst must not
 * overlap.  Same stream, ownership and error rules as migemm_gemm; rows == 0
 * or cols == 0 is a no-op.
 */
int migemm_convert(int src_dtype, int dst_dtype, int64_t rows, int64_t cols,
                   const void* src, int64_t lds, void* dst, int64_t ldd, void* stream);

/* Number of variants (they are numbered 0 .. count-1). */
int migemm_variant_count(void);

/* Short name of a variant, or NULL for an unknown index.  Static storage. */
const char* migemm_variant_name(int variant);

/* 1 if the variant takes this dtype, 0 if not (or if either is unknown). */
int migemm_variant_supports(int variant, int dtype);

/* Number of tile configurations of a variant (0 for an unknown index). */
int migemm_config_count(int variant);

/* Name of a configuration ("256x256x64 8w 16x16x32" ...), or NULL.  Static storage. */
const char* migemm_config_name(int variant, int config);

/*
 * The selection for these arguments without launching anything: writes the
 * variant and config indices migemm_gemm would use.  Same argument checks as
 * migemm_gemm (pointers are only inspected for alignment and may be NULL).
 */
int migemm_select(int64_t M, int64_t N, int64_t K, int dtype,
                  const void* A, int64_t lda, const void* B, int64_t ldb,
                  const float* C, int64_t ldc, int* variant, int* config);

/* Text of a status code.  Static storage. */
const char* migemm_status_string(int status);

/* The hipError_t code behind the calling thread's last MIGEMM_ERR_HIP (0 if none). */
int migemm_last_hip_error(void);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int migemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MIGEMM_H */
