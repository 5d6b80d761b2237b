// tdg_probe.hip -- the measured compute ceiling: a kernel that issues only
// MFMAs, the same instructions the GEMM's tile micro-kernel issues, with no
// memory traffic.  Its rate is the denominator that the chip actually
// sustains ("Analyze Kernel Bottleneck", Step 2: compare achieved
// throughput with what the hardware delivers, not only with the data-sheet
// peak).  On MI355X the data-sheet rate needs 2.4 GHz; under full MFMA load
// the chip's power limit holds the clock lower, and by how much depends on
// the operand bits, so the operands here change every step like a GEMM's
// do: four pseudo-random operand sets per lane, rotated through the eight
// independent accumulator chains of each wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tdg_internal.h"
#include "tdgemm.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int PROBE_THREADS = 256;      // one wave per SIMD
constexpr int PROBE_WG_PER_CU = 2;      // two waves per SIMD, like the 8-wave GEMM tile
constexpr int PROBE_CUS = 256;

__device__ __forceinline__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// Operand words: random binary16 pairs or binary32 values with exponents
// near 1.0 (no infinities or NaNs), or random bytes for INT8.
__device__ __forceinline__ uint32_t operand_word(int dtype, uint32_t seed) {
    const uint32_t r = mix(seed);
    if (dtype == TDG_DTYPE_I8I32) return r;
    if (dtype == TDG_DTYPE_F32F32) return (r & 0x807FFFFFu) | 0x3F000000u;  // 0.5 .. 1
    return (r & 0x83FF83FFu) | 0x38003800u;  // sign, mantissa random; exponent 14 (0.5 .. 1)
}

template <int DT>
__global__ void __launch_bounds__(PROBE_THREADS) k_mfma_probe(int64_t iters, float *sink) {
    const uint32_t lane = threadIdx.x + blockIdx.x * PROBE_THREADS;
    i32x4 a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; s++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            a[s][e] = (int)operand_word(DT, lane * 32u + s * 8u + e);
            b[s][e] = (int)operand_word(DT, lane * 32u + s * 8u + 4u + e);
        }
    float total = 0.0f;
    if constexpr (DT == TDG_DTYPE_F16F32) {
        f32x16 c[8];
#pragma unroll
        for (int k = 0; k < 8; k++) c[k] = f32x16{};
        for (int64_t it = 0; it < iters; it += 4) {
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int k = 0; k < 8; k++)
                    c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(f16x8, a[(k + u) & 3]), __builtin_bit_cast(f16x8, b[(k + 1) & 3]),
                        c[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int v = 0; v < 16; v++) total += c[k][v];
    } else if constexpr (DT == TDG_DTYPE_F32F32) {
        f32x16 c[8];
#pragma unroll
        for (int k = 0; k < 8; k++) c[k] = f32x16{};
        for (int64_t it = 0; it < iters; it += 4) {
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    // through scalars: a bit cast of a vector subscript reads element 0
                    const uint32_t x = (uint32_t)a[(k + u) & 3][u], y = (uint32_t)b[(k + 1) & 3][k & 3];
                    c[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, x),
                                                                __builtin_bit_cast(float, y), c[k], 0, 0, 0);
                }
        }
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int v = 0; v < 16; v++) total += c[k][v];
    } else {
        i32x16 c[8];
#pragma unroll
        for (int k = 0; k < 8; k++) c[k] = i32x16{};
        for (int64_t it = 0; it < iters; it += 4) {
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int k = 0; k < 8; k++)
                    c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(k + u) & 3], b[(k + 1) & 3], c[k], 0, 0, 0);
        }
        int t = 0;
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int v = 0; v < 16; v++) t += c[k][v];
        total = (float)t;
    }
    sink[lane] = total;  // keeps the chains live
}

}  // namespace

extern "C" {

static bool probe_dtype(int dtype) {
    return dtype == TDG_DTYPE_F16F32 || dtype == TDG_DTYPE_I8I32 || dtype == TDG_DTYPE_F32F32;
}

int64_t tdg_mfma_probe_ops(int dtype, int64_t iters) {
    if (!probe_dtype(dtype) || iters < 0 || iters % 4) return -1;
    const int64_t k = dtype == TDG_DTYPE_F16F32 ? 16 : (dtype == TDG_DTYPE_I8I32 ? 32 : 2);
    const int64_t waves = (int64_t)PROBE_CUS * PROBE_WG_PER_CU * (PROBE_THREADS / 64);
    return 2 * 32 * 32 * k * 8 * iters * waves;
}

int64_t tdg_mfma_probe_sink_floats(void) {
    return (int64_t)PROBE_CUS * PROBE_WG_PER_CU * PROBE_THREADS;
}

int tdg_mfma_probe(int dtype, int64_t iters, float *sink, void *stream) {
    if (!probe_dtype(dtype)) return TDG_ERR_INVALID_ARG;
    if (iters < 0 || iters % 4 || !sink) return TDG_ERR_INVALID_ARG;
    const int dev = tdg::device_check();
    if (dev != TDG_OK) return dev;
    void *kargs[] = {&iters, &sink};
    const void *fn = dtype == TDG_DTYPE_F16F32 ? (const void *)&k_mfma_probe<TDG_DTYPE_F16F32>
                     : dtype == TDG_DTYPE_I8I32 ? (const void *)&k_mfma_probe<TDG_DTYPE_I8I32>
                                                : (const void *)&k_mfma_probe<TDG_DTYPE_F32F32>;
    if (hipLaunchKernel(fn, dim3(PROBE_CUS * PROBE_WG_PER_CU), dim3(PROBE_THREADS), kargs, 0,
                        (hipStream_t)stream) != hipSuccess)
        return TDG_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return TDG_ERR_LAUNCH;
    return TDG_OK;
}

}  // extern "C"
