// tdg_noalloc.hip -- split K with no allocation at all, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The gemm_*_splitk entry points take their partial products in a workspace
// the caller passes.  gemm_splitk_noalloc takes them in `scratch`, a
// file-scope device array of TDG_NOALLOC_SCRATCH_BYTES.  Each GPU the
// library runs on holds its own copy of the array, at its own address, from
// the first use of this code object on that GPU until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// address must never reach a kernel.  The device address is asked of the
// runtime once per device (hipGetSymbolAddress, with that device current) and
// kept; only that address is passed on.
//
// Every call on one GPU shares that GPU's array.  Calls that overlap in time
// on one GPU (different streams, or host threads) race on it; calls enqueued
// on one stream do not.  Nothing in the array has to start at zero: each part
// writes every element of its M x N partial product before the summation
// kernel, enqueued after it on the same stream, reads it.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "tdg_internal.h"
#include "tdgemm.h"

namespace {

static __device__ __align__(256) unsigned char scratch[TDG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device; NULL until asked

// The device address of the current device's `scratch` (asked of the runtime
// on the first call on each device), or NULL when the runtime cannot say.
void *scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int gemm_splitk_noalloc(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                                   const void *B, int64_t ldb, void *C, int64_t ldc, int parts,
                                   void *stream) {
    // Everything checkable on the host is checked before any HIP call.
    int rc = tdg::validate_gemm(dtype, M, N, K, A, lda, B, ldb, C, ldc);
    if (rc != TDG_OK) return rc;
    if (parts < 0) return TDG_ERR_INVALID_ARG;
    if (parts > 1 && tdg::splitk_bytes(parts, M, N) > (uint64_t)TDG_NOALLOC_SCRATCH_BYTES)
        return TDG_ERR_SCRATCH;
    if (M == 0 || N == 0) return TDG_OK;
    rc = tdg::device_check();
    if (rc != TDG_OK) return rc;
    void *ws = scratch_address();
    if (!ws) return TDG_ERR_LAUNCH;
    return tdg::run_splitk(dtype, M, N, K, A, lda, B, ldb, C, ldc, parts, ws, TDG_NOALLOC_SCRATCH_BYTES,
                           stream, TDG_NOALLOC_SCRATCH_BYTES);
}
