// noalloc.hip -- migemm_gemm_noalloc: the general product for callers that
// cannot allocate device memory or lend a workspace (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// It is migemm_gemm_ws with the workspace taken from `scratch`, a file-scope
// device array of fixed size that every GPU the library runs on holds from the
// time the library's code object is loaded there until the process ends.  The
// device address of each GPU's copy is looked up once per device (with that
// device current) and kept; host code passes that address, never the array's
// name, to the kernels.  No allocating call is made.
//
// Calls on one GPU share its array, which keeps the last call's contents: its
// users (the copies of FP16/BF16 and INT8 operands, which write whole rows,
// zero padding included, and split-K, whose slices each write their whole
// M x N block of sums before the sum kernel reads them) overwrite every byte
// they read, so nothing needs clearing.  Calls that overlap in time on one GPU
// (two streams, or two host threads) race on the array.
#include <mutex>

#include "common.hpp"
#include "migemm.h"

namespace migemm {
namespace {

constexpr int64_t kScratchBytes = int64_t(64) << 20;  // 64 MiB per GPU

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

// The device address of the current device's copy of `scratch`, looked up on
// the first call on that device.
hipError_t scratch_on_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev]() {
        void* p = nullptr;
        g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_lookup[dev] == hipSuccess ? p : nullptr;
    });
    *ptr = g_scratch[dev];
    return g_lookup[dev];
}

}  // namespace
}  // namespace migemm

using namespace migemm;

extern "C" int migemm_gemm_noalloc(int variant, int config, int op_a, int op_b, int64_t M,
                                   int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                                   const void* B, int64_t ldb, float alpha, float beta,
                                   int c_dtype, void* C, int64_t ldc, void* stream) {
    int64_t need = 0;
    int st = workspace_bytes(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, &need);
    if (st != MIGEMM_OK) return st;
    if (need > kScratchBytes) return MIGEMM_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = scratch_on_current_device(&ws);
        if (e != hipSuccess || ws == nullptr) {
            (void)hipGetLastError();
            return MIGEMM_ERR_HIP;
        }
    }
    return run_gemm(variant, config, op_a, op_b, M, N, K, dtype, A, lda, B, ldb, alpha, beta,
                    c_dtype, C, ldc, ws, need > 0 ? kScratchBytes : 0, stream);
}
