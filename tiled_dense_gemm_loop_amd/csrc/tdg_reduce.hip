// tdg_reduce.hip -- the second pass of a split-K product: C = sum over the
// K parts of the partial C tiles the GEMM kernel wrote to the workspace.
//
// The workspace holds `parts` dense M x N partial products (row length N),
// part p at workspace + p * M * N elements.  Each output element is summed in
// part order 0, 1, ..., parts - 1, so the result does not depend on how the
// work was scheduled (FP32: one fixed rounding sequence; INT32: exact, with
// the wrap-around of 32-bit addition).  The pass reads parts * M * N * 4
// bytes and writes M * N * 4: it is bound by HBM, so it moves 16 bytes per
// lane where the rows allow it (N and ldc multiples of 4, C 16-byte aligned)
// and 4 bytes otherwise.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tdg_internal.h"
#include "tdgemm.h"

namespace {

constexpr int THREADS = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T, typename V>
__global__ void __launch_bounds__(THREADS) k_sum_parts(const T *__restrict__ ws, int parts, int M, int N,
                                                      T *__restrict__ C, int64_t ldc, int vec) {
    const int64_t part = (int64_t)M * N;
    if (vec) {
        // element 4q .. 4q + 3 of the dense M x N layout; a group never
        // crosses a row because N is a multiple of 4
        const int64_t groups = part / 4;
        for (int64_t q = (int64_t)blockIdx.x * THREADS + threadIdx.x; q < groups;
             q += (int64_t)gridDim.x * THREADS) {
            V s = *(const V *)(ws + 4 * q);
            for (int p = 1; p < parts; p++) s += *(const V *)(ws + (int64_t)p * part + 4 * q);
            const int64_t i = (4 * q) / N, j = (4 * q) - i * N;
            *(V *)(C + i * ldc + j) = s;
        }
    } else {
        for (int64_t q = (int64_t)blockIdx.x * THREADS + threadIdx.x; q < part;
             q += (int64_t)gridDim.x * THREADS) {
            T s = ws[q];
            for (int p = 1; p < parts; p++) s += ws[(int64_t)p * part + q];
            const int64_t i = q / N, j = q - i * N;
            C[i * ldc + j] = s;
        }
    }
}

}  // namespace

namespace tdg {

int launch_sum_parts(int dtype, int parts, const void *ws, int64_t M, int64_t N, void *C, int64_t ldc,
                     void *stream) {
    const bool vec = N % 4 == 0 && ldc % 4 == 0 && (uintptr_t)C % 16 == 0 && (uintptr_t)ws % 16 == 0;
    const int64_t work = vec ? M * N / 4 : M * N;
    int64_t blocks = (work + THREADS - 1) / THREADS;
    if (blocks > 4096) blocks = 4096;  // grid-stride beyond 16 waves per CU
    if (blocks < 1) blocks = 1;
    int m = (int)M, n = (int)N, v = vec ? 1 : 0;
    void *kargs[] = {&ws, &parts, &m, &n, &C, &ldc, &v};
    // INT32 parts are summed as unsigned words: the same bits as the
    // matrix cores' wrapping 32-bit accumulation, without signed overflow
    const void *fn = dtype == TDG_DTYPE_I8I32 ? (const void *)&k_sum_parts<uint32_t, u32x4>
                                              : (const void *)&k_sum_parts<float, f32x4>;
    if (hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(THREADS), kargs, 0, (hipStream_t)stream) !=
        hipSuccess)
        return TDG_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return TDG_ERR_LAUNCH;
    return TDG_OK;
}

}  // namespace tdg
