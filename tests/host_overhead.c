/* Host time of the C ABI's entry checks and configuration selection, without a
 * GPU: migemm_select runs the validation and the selection table that every
 * product call runs before it launches (the launch itself aside), and
 * migemm_workspace_size adds the packed path's size rule.  Shapes from 256^3 to
 * 8192^3, aligned and ragged, FP32, FP16, BF16 and INT8, every layout through
 * migemm_workspace_size.  Prints the mean nanoseconds per call of each. */
#include <stdint.h>
#include <stdio.h>
#include <time.h>

#include "migemm.h"

static double now_ns(void) {
    struct timespec t;
    clock_gettime(CLOCK_MONOTONIC, &t);
    return (double)t.tv_sec * 1e9 + (double)t.tv_nsec;
}

int main(void) {
    /* M, N, K, dtype (pointers stand for 256-byte aligned buffers) */
    static const int64_t shapes[][4] = {
        {256, 256, 256, MIGEMM_F16},    {1024, 1024, 1024, MIGEMM_F32},
        {1024, 1024, 1024, MIGEMM_F16}, {2048, 2048, 2048, MIGEMM_BF16},
        {2050, 2047, 2056, MIGEMM_F16}, {8192, 8192, 8192, MIGEMM_BF16},
        {4096, 4096, 4096, MIGEMM_F32}, {8200, 8192, 8192, MIGEMM_I8},
    };
    const int ns = (int)(sizeof(shapes) / sizeof(shapes[0]));
    const void* A = (const void*)(uintptr_t)0x100000000ull;
    const void* B = (const void*)(uintptr_t)0x200000000ull;
    const float* C = (const float*)(uintptr_t)0x300000000ull;
    const int reps = 20000;
    volatile int sink = 0;
    double t0 = now_ns();
    for (int r = 0; r < reps; ++r)
        for (int i = 0; i < ns; ++i) {
            int v = 0, c = 0;
            const int64_t M = shapes[i][0], N = shapes[i][1], K = shapes[i][2];
            sink += migemm_select(M, N, K, (int)shapes[i][3], A, K, B, N, C, N, &v, &c) + v + c;
        }
    const double select_ns = (now_ns() - t0) / ((double)reps * ns);
    t0 = now_ns();
    for (int r = 0; r < reps; ++r)
        for (int i = 0; i < ns; ++i) {
            int64_t bytes = 0;
            const int64_t M = shapes[i][0], N = shapes[i][1], K = shapes[i][2];
            const int op = r & 3;
            const int64_t lda = (op & 1) ? M : K, ldb = (op & 2) ? K : N;
            sink += migemm_workspace_size(MIGEMM_VARIANT_AUTO, -1, op & 1, op >> 1, M, N, K,
                                          (int)shapes[i][3], A, lda, B, ldb, &bytes) +
                    (int)(bytes & 1);
        }
    const double ws_ns = (now_ns() - t0) / ((double)reps * ns);
    printf("select_ns %.1f\nworkspace_size_ns %.1f\nsink %d\n", select_ns, ws_ns, sink & 1);
    return 0;
}
