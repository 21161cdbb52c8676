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
