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

// LDS read rate.  One workgroup of 8 waves per CU (2 per SIMD, like the
// 8-wave GEMM tile) reads its 64 KiB LDS buffer in a loop: 16-byte reads
// (ds_read_b128, the A fragments), transposing 8-byte reads
// (ds_read_b64_tr_b16, the B fragments) or plain 8-byte reads
// (ds_read_b64).  Lane l reads 16 (or 8) bytes at l * 16 within a 1 KiB
// row, and waves and reads move over the 64 rows, so no two lanes of a read
// share a bank.  The loads are volatile (or intrinsics the compiler does not
// merge), so every one issues.  Each workgroup writes its shader cycles
// (s_memtime) to out[blockIdx], and a value of its reads to
// out[PROBE_CUS + blockIdx], which keeps them live.
constexpr int LDS_PROBE_THREADS = 512;
constexpr int LDS_PROBE_BYTES = 65536;
constexpr int LDS_PROBE_UNROLL = 8;

template <int MODE>
__global__ void __launch_bounds__(LDS_PROBE_THREADS) k_lds_probe(int64_t iters, uint32_t *out) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_PROBE_BYTES];
    typedef __attribute__((address_space(3))) unsigned char lds_byte;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid * 16; i < LDS_PROBE_BYTES; i += LDS_PROBE_THREADS * 16)
        *(u32x4 *)(lds + i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
    __syncthreads();
    lds_byte *base = (lds_byte *)lds + lane * 16;
    uint32_t acc = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int64_t it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < LDS_PROBE_UNROLL; j++) {
            const int row = (int)(((it * LDS_PROBE_UNROLL + j) * 8 + wave) & 63);
            lds_byte *p = base + row * 1024;
            if constexpr (MODE == 0) {
                const u32x4 v = *(volatile const __attribute__((address_space(3))) u32x4 *)p;
                acc ^= v[0] ^ v[3];
            } else if constexpr (MODE == 1) {
                const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)p);
                acc ^= (uint32_t)(uint16_t)v[0] ^ (uint32_t)(uint16_t)v[3];
            } else {
                const i16x4 v = *(volatile const __attribute__((address_space(3))) i16x4 *)p;
                acc ^= (uint32_t)(uint16_t)v[0] ^ (uint32_t)(uint16_t)v[3];
            }
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if (tid == 0) {
        out[blockIdx.x] = (uint32_t)(t1 - t0);
        out[PROBE_CUS + blockIdx.x] = acc;
    }
}

}  // namespace

extern "C" {

int64_t tdg_lds_probe_bytes(int mode, int64_t iters) {
    if (mode < 0 || mode > 2 || iters < 0) return -1;
    return iters * LDS_PROBE_UNROLL * LDS_PROBE_THREADS * (mode == 0 ? 16 : 8);
}

int tdg_lds_probe(int mode, int64_t iters, uint32_t *out, void *stream) {
    if (mode < 0 || mode > 2 || iters < 0 || !out) return TDG_ERR_INVALID_ARG;
    const int dev = tdg::device_check();
    if (dev != TDG_OK) return dev;
    void *kargs[] = {&iters, &out};
    const void *fn = mode == 0 ? (const void *)&k_lds_probe<0>
                     : mode == 1 ? (const void *)&k_lds_probe<1>
                                 : (const void *)&k_lds_probe<2>;
    if (hipLaunchKernel(fn, dim3(PROBE_CUS), dim3(LDS_PROBE_THREADS), kargs, 0, (hipStream_t)stream) !=
        hipSuccess)
        return TDG_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return TDG_ERR_LAUNCH;
    return TDG_OK;
}

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
