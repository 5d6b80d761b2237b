// tdg_internal.h -- declarations shared by the kernel table and the host API.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace tdg {

// One built kernel: its tile shape, loop form and launch needs.
struct KernelEntry {
    int dtype;      // 0 = FP16 -> FP32, 1 = INT8 -> INT32, 2 = FP32 -> FP32
    int bm, bn;     // C tile
    int bkb;        // K tile in bytes per row (BK = bkb / sizeof(T))
    int wm, wn;     // wave grid; waves = wm * wn
    int stages;     // LDS buffers
    int variant;    // 1 sequential, 2 register prefetch, 3 direct-to-LDS
    bool guard;     // bounds-checked loads and stores
    const void *fn; // __global__ function
    int threads;    // workgroup size
    int lds_bytes;  // static LDS per workgroup
};

// Per-dtype tables (one translation unit each) and their concatenation.
const KernelEntry *kernel_table_f16(int *count);
const KernelEntry *kernel_table_i8(int *count);
const KernelEntry *kernel_table_f32(int *count);
const KernelEntry *kernel_table(int *count);

// TDG_OK when the current device is gfx950, else TDG_ERR_NO_DEVICE.
int device_check();

// Split-K second pass: C (M x N, ldc) = sum over `parts` dense M x N partial
// products at ws, in part order.  FP32 for the FP16 / FP32 dtypes, INT32 for
// INT8.  Enqueued on `stream`.
int launch_sum_parts(int dtype, int parts, const void *ws, int64_t M, int64_t N, void *C, int64_t ldc,
                     void *stream);

// Bytes of `parts` dense M x N partial products of 4 bytes, or UINT64_MAX
// when that does not fit in 64 bits (0 <= M, N < 2^31, so one product's
// M * N * 4 always does; a caller's part count can still carry it over).
uint64_t splitk_bytes(int64_t parts, int64_t M, int64_t N);

// Argument validation of a GEMM call (TDG_OK or TDG_ERR_INVALID_ARG); no
// HIP call.
int validate_gemm(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                  int64_t ldb, const void *C, int64_t ldc);

// Split K into the workspace ws of ws_bytes bytes (the gemm_*_splitk entry
// points).  With parts == 0 the planner chooses the count, among the counts
// whose partial products take at most auto_limit bytes.
int run_splitk(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
               int64_t ldb, void *C, int64_t ldc, int parts, void *ws, size_t ws_bytes, void *stream,
               uint64_t auto_limit = UINT64_MAX);

}  // namespace tdg
