// convert.hip -- element-type conversion of a matrix on the device: FP32, FP16
// and BF16 in any pairing, round to nearest even where the target is narrower
// (page "04-wmma-matmul.cu", the FP32 -> half conversion before the product;
// page "CUDA-Practice 09", section on mixed precision: 16-bit inputs halve the
// bytes the product reads).  This is the step before the product for callers
// whose data are FP32 and who want the 16-bit matrix-core path.
//
// Memory-bound: each element is read once and written once.  A work-item
// converts 8 consecutive elements of a row: one 16-byte load of 16-bit source
// (two of FP32) and one 16-byte store of 16-bit target (two of FP32) when
// both rows are 16-byte aligned; element-wise otherwise and at row ends.
// Workgroups stride over the rows' 8-element pieces, so any shape is covered
// by a grid sized to the chip.
#include "common.hpp"

namespace migemm {
namespace {

// One element to and from FP32 (every FP16 and BF16 value is exact in FP32;
// the narrowing stores round to nearest even), and the same for 8 elements
// held as 16-byte words (two words of FP32, one of a 16-bit type; 16-bit
// element 2i in the low half of 32-bit word i).
template <typename T> struct Conv;
template <> struct Conv<float> {
    static constexpr int WORDS = 2;
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
    static __device__ __forceinline__ void unpack(const u32x4 (&w)[2], float (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i / 4][i % 4]);
    }
    static __device__ __forceinline__ void pack(const float (&v)[8], u32x4 (&w)[2]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i / 4][i % 4] = __float_as_uint(v[i]);
    }
};
template <> struct Conv<_Float16> {
    static constexpr int WORDS = 1;
    static __device__ __forceinline__ float load(const _Float16* p) { return static_cast<float>(*p); }
    static __device__ __forceinline__ void store(_Float16* p, float v) { *p = static_cast<_Float16>(v); }
    static __device__ __forceinline__ float half_bits(uint32_t b) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
    }
    static __device__ __forceinline__ uint32_t bits(float v) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
    static __device__ __forceinline__ void unpack(const u32x4 (&w)[1], float (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = half_bits(w[0][i] & 0xffffu);
            v[2 * i + 1] = half_bits(w[0][i] >> 16);
        }
    }
    static __device__ __forceinline__ void pack(const float (&v)[8], u32x4 (&w)[1]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[0][i] = bits(v[2 * i]) | (bits(v[2 * i + 1]) << 16);
    }
};
template <> struct Conv<bf16_t> {
    static constexpr int WORDS = 1;
    static __device__ __forceinline__ float load(const bf16_t* p) { return to_f32(*p); }
    static __device__ __forceinline__ void store(bf16_t* p, float v) { p->bits = f32_to_bf16_bits(v); }
    static __device__ __forceinline__ void unpack(const u32x4 (&w)[1], float (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[0][i] << 16);
            v[2 * i + 1] = __uint_as_float(w[0][i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void pack(const float (&v)[8], u32x4 (&w)[1]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[0][i] = static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i])) |
                      (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i + 1])) << 16);
    }
};

template <typename S, typename D>
__global__ __launch_bounds__(256) void convert_kernel(int64_t rows, int64_t cols,
                                                      const S* __restrict__ src, int64_t lds,
                                                      D* __restrict__ dst, int64_t ldd,
                                                      bool vec) {
    const int64_t pieces = ceil_div(cols, 8);
    const int64_t total = rows * pieces;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t r = e / pieces, c0 = (e % pieces) * 8;
        const S* ps = src + r * lds + c0;
        D* pd = dst + r * ldd + c0;
        if (vec && c0 + 8 <= cols) {
            u32x4 in[Conv<S>::WORDS], out[Conv<D>::WORDS];
#pragma unroll
            for (int w = 0; w < Conv<S>::WORDS; ++w) in[w] = reinterpret_cast<const u32x4*>(ps)[w];
            float v[8];
            Conv<S>::unpack(in, v);
            Conv<D>::pack(v, out);
#pragma unroll
            for (int w = 0; w < Conv<D>::WORDS; ++w) reinterpret_cast<u32x4*>(pd)[w] = out[w];
        } else {
            for (int i = 0; i < 8 && c0 + i < cols; ++i) Conv<D>::store(pd + i, Conv<S>::load(ps + i));
        }
    }
}

template <typename S, typename D>
hipError_t launch_pair(int64_t rows, int64_t cols, const void* src, int64_t lds, void* dst,
                       int64_t ldd, hipStream_t s) {
    const bool vec = aligned16(src) && aligned16(dst) && (lds * sizeof(S)) % 16 == 0 &&
                     (ldd * sizeof(D)) % 16 == 0;
    int64_t blocks = ceil_div(rows * ceil_div(cols, 8), 256);
    if (blocks > 65536) blocks = 65536;  // beyond this the loop strides over the rest
    convert_kernel<S, D><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
        rows, cols, static_cast<const S*>(src), lds, static_cast<D*>(dst), ldd, vec);
    return hipGetLastError();
}

template <typename S>
hipError_t launch_from(int dst_dtype, int64_t rows, int64_t cols, const void* src, int64_t lds,
                       void* dst, int64_t ldd, hipStream_t s) {
    switch (dst_dtype) {
        case 0: return launch_pair<S, float>(rows, cols, src, lds, dst, ldd, s);
        case 1: return launch_pair<S, _Float16>(rows, cols, src, lds, dst, ldd, s);
        default: return launch_pair<S, bf16_t>(rows, cols, src, lds, dst, ldd, s);
    }
}

}  // namespace

hipError_t launch_convert(int src_dtype, int dst_dtype, int64_t rows, int64_t cols,
                          const void* src, int64_t lds, void* dst, int64_t ldd, hipStream_t s) {
    switch (src_dtype) {
        case 0: return launch_from<float>(dst_dtype, rows, cols, src, lds, dst, ldd, s);
        case 1: return launch_from<_Float16>(dst_dtype, rows, cols, src, lds, dst, ldd, s);
        default: return launch_from<bf16_t>(dst_dtype, rows, cols, src, lds, dst, ldd, s);
    }
}

}  // namespace migemm
