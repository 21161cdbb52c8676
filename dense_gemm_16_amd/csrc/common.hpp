// common.hpp -- internal types shared by the kernels and the C ABI of the
// gfx950 GEMM library.  Not installed; the public interface is migemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace migemm {

// Arguments of one product, already validated by the C ABI.
struct GemmArgs {
    int64_t M, N, K;
    int dtype;
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    float* C;
    int64_t ldc;
    hipStream_t stream;
};

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

template <typename T> struct ZeroOf { static __device__ __forceinline__ T get() { return T(0); } };
template <> struct ZeroOf<bf16_t> {
    static __device__ __forceinline__ bf16_t get() { return bf16_t{0}; }
};

// 16-byte vector of raw bits (the unit of global and LDS traffic).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
hipError_t launch_zero_fill(float* C, int64_t M, int64_t N, int64_t ldc, hipStream_t s);

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

}  // namespace migemm
