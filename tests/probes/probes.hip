// probes.hip -- test-only kernels that pin the lane semantics of the gfx950
// instructions the GEMM kernels rely on, and a matrix-core throughput probe.
// Every access is in bounds: the semantic probes run as one 64-lane wavefront
// over fixed-size buffers; the throughput probe writes one float per thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

// ds_read_b64_tr_b16: LDS holds lds[i] = i (4096 16-bit words); lane l reads the
// 8-byte word at byte offset addr[l] (a multiple of 8 below 8192) with transpose.
__global__ __launch_bounds__(64) void tr16_kernel(const int* addr, uint16_t* out) {
    __shared__ uint16_t lds[4096];
    for (int i = threadIdx.x; i < 4096; i += 64) lds[i] = static_cast<uint16_t>(i);
    __syncthreads();
    const int a = addr[threadIdx.x] & 8184;  // in bounds whatever the host passed
    // address-space casts must be C-style casts in HIP
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)lds + a));
    for (int e = 0; e < 4; ++e) out[threadIdx.x * 4 + e] = static_cast<uint16_t>(v[e]);
}

// ds_read_b64_tr_b8: LDS holds 8192 bytes, byte i = (mode == 0 ? i & 255 : i >> 8);
// lane l reads the 8-byte word at byte offset addr[l] (a multiple of 8 below
// 8192) with transpose.  The two modes together give the source offset of every
// byte a lane receives.
typedef int i32x2v __attribute__((ext_vector_type(2)));
__global__ __launch_bounds__(64) void tr8_kernel(const int* addr, uint8_t* out, int mode) {
    __shared__ uint8_t lds[8192];
    for (int i = threadIdx.x; i < 8192; i += 64)
        lds[i] = static_cast<uint8_t>(mode == 0 ? (i & 255) : (i >> 8));
    __syncthreads();
    const int a = addr[threadIdx.x] & 8184;  // in bounds whatever the host passed
    i32x2v v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2v*)((LDS_AS char*)lds + a));
    for (int e = 0; e < 8; ++e)
        out[threadIdx.x * 8 + e] = static_cast<uint8_t>(static_cast<uint32_t>(v[e / 4]) >> (8 * (e % 4)));
}

// global_load_lds_dwordx4: lane l loads the 16 bytes at src + 4*off[l] dwords
// (off[l] < 64) into LDS at a base of 64 dwords; the whole 1024-dword LDS array
// (pre-filled with 0xffffffff) is copied out.
__global__ __launch_bounds__(64) void lds_load_kernel(const uint32_t* src, const int* off,
                                                      uint32_t* out) {
    __shared__ uint32_t lds[1024];
    for (int i = threadIdx.x; i < 1024; i += 64) lds[i] = 0xffffffffu;
    __syncthreads();
    const int o = (off[threadIdx.x] & 63) * 4;
    __builtin_amdgcn_global_load_lds(src + o, (LDS_AS void*)(lds + 64), 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = threadIdx.x; i < 1024; i += 64) out[i] = lds[i];
}

extern "C" int probe_tr8(const int* addr, uint8_t* out, int mode, void* stream) {
    tr8_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(addr, out, mode);
    return static_cast<int>(hipGetLastError());
}

extern "C" int probe_tr16(const int* addr, uint16_t* out, void* stream) {
    tr16_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(addr, out);
    return static_cast<int>(hipGetLastError());
}

extern "C" int probe_lds_load(const uint32_t* src, const int* off, uint32_t* out, void* stream) {
    lds_load_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(src, off, out);
    return static_cast<int>(hipGetLastError());
}

// Matrix-core throughput with no memory traffic: every wave runs 8 independent
// accumulator chains of one MFMA shape for `iters` rounds, from operands held in
// registers.  mode 0: zero operands; 1: all ones; 2: hashed values in [-0.5, 0.5)
// (random bits, as GEMM inputs have).  Each thread stores the sum of its
// accumulators, so for mode 1 every output is 8 * R * iters * k (R accumulator
// registers per lane, k the instruction's depth).  512 threads per workgroup: two
// waves per SIMD, as in the GEMM kernels.
typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));
typedef float probe_f32x4 __attribute__((ext_vector_type(4)));

template <int MF>
__global__ __launch_bounds__(512) void mfma_ceiling_kernel(float* out, int iters, int mode) {
    using Acc = typename std::conditional<MF == 32, probe_f32x16, probe_f32x4>::type;
    constexpr int NACC = 8;
    Acc acc[NACC];
    for (int i = 0; i < NACC; ++i) acc[i] = Acc{};
    probe_bf16x8 a[2], b[2];
    for (int v = 0; v < 2; ++v)
        for (int e = 0; e < 8; ++e) {
            uint32_t h = (threadIdx.x * 8u + e + v * 977u) * 2654435761u ^ (blockIdx.x * 40503u);
            h ^= h >> 13;
            h *= 0x5bd1e995u;
            h ^= h >> 15;
            float x = mode == 0 ? 0.0f : mode == 1 ? 1.0f : (float)(h & 0xffff) / 65536.0f - 0.5f;
            float y = mode == 0 ? 0.0f : mode == 1 ? 1.0f : (float)(h >> 16) / 65536.0f - 0.5f;
            a[v][e] = (__bf16)x;
            b[v][e] = (__bf16)y;
        }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < NACC; ++i) {
            if constexpr (MF == 32)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i & 1], b[(i >> 1) & 1], acc[i], 0, 0, 0);
            else
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i & 1], b[(i >> 1) & 1], acc[i], 0, 0, 0);
        }
    }
    float s = 0.f;
    for (int i = 0; i < NACC; ++i)
        for (int r = 0; r < (MF == 32 ? 16 : 4); ++r) s += acc[i][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// out holds blocks * 512 floats.
extern "C" int probe_mfma_ceiling(int mf, float* out, int blocks, int iters, int mode, void* stream) {
    if ((mf != 16 && mf != 32) || blocks <= 0 || iters <= 0 || mode < 0 || mode > 2) return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mf == 32)
        mfma_ceiling_kernel<32><<<blocks, 512, 0, s>>>(out, iters, mode);
    else
        mfma_ceiling_kernel<16><<<blocks, 512, 0, s>>>(out, iters, mode);
    return static_cast<int>(hipGetLastError());
}
