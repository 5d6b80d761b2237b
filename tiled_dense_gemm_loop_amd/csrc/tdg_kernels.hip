// tdg_kernels.hip -- the built-in kernel configurations and their table.
//
// Each tile shape (BM x BN, K tile of BKB bytes, WM x WN waves) is built for
// both dtypes in seven forms: the sequential baseline, the register-prefetch
// loop with one and with two LDS buffers, the direct-to-LDS loop, and the
// bounds-checked forms of the baseline, of the double-buffered
// register-prefetch loop (any ragged or misaligned operands) and of the
// direct-to-LDS loop (ragged shapes with aligned, whole-chunk rows).
#include "tdg_internal.h"
#include "tdg_kernels.hpp"

namespace tdg {

#define TDG_ENTRY(DT, BM, BN, BKB, WM, WN, ST, VAR, GUARD)                                        \
    KernelEntry{DT, BM, BN, BKB, WM, WN, ST, VAR, GUARD,                                         \
                (const void *)&tdg_gemm_kernel<DT, BM, BN, BKB, WM, WN, ST, VAR, GUARD>,         \
                WM * WN * 64, ST * Geo<DT, BM, BN, BKB, WM, WN>::STAGE_BYTES}

#define TDG_SHAPE(DT, BM, BN, BKB, WM, WN)                                  \
    TDG_ENTRY(DT, BM, BN, BKB, WM, WN, 1, VAR_SINGLE, false),               \
        TDG_ENTRY(DT, BM, BN, BKB, WM, WN, 1, VAR_REG, false),              \
        TDG_ENTRY(DT, BM, BN, BKB, WM, WN, 2, VAR_REG, false),              \
        TDG_ENTRY(DT, BM, BN, BKB, WM, WN, 2, VAR_DIRECT, false),           \
        TDG_ENTRY(DT, BM, BN, BKB, WM, WN, 1, VAR_SINGLE, true),            \
        TDG_ENTRY(DT, BM, BN, BKB, WM, WN, 2, VAR_REG, true),               \
        TDG_ENTRY(DT, BM, BN, BKB, WM, WN, 2, VAR_DIRECT, true)

// Deeper direct-to-LDS rings where the LDS budget allows.
#define TDG_DIRECT(DT, BM, BN, BKB, WM, WN, ST) TDG_ENTRY(DT, BM, BN, BKB, WM, WN, ST, VAR_DIRECT, false)
// ... and their bounds-checked forms, for every ring the planner's table
// can pick, so that a ragged shape keeps the ring of its aligned neighbour.
#define TDG_DIRECT_G(DT, BM, BN, BKB, WM, WN, ST) TDG_ENTRY(DT, BM, BN, BKB, WM, WN, ST, VAR_DIRECT, true)

#define TDG_SHAPES(DT)                                                                   \
    TDG_SHAPE(DT, 256, 256, 128, 2, 2), TDG_SHAPE(DT, 256, 256, 128, 2, 4),              \
        TDG_SHAPE(DT, 256, 256, 64, 2, 2), TDG_DIRECT(DT, 256, 256, 64, 2, 2, 3),        \
        TDG_DIRECT(DT, 256, 256, 64, 2, 2, 4), TDG_SHAPE(DT, 256, 256, 64, 2, 4),        \
        TDG_DIRECT(DT, 256, 256, 64, 2, 4, 3), TDG_DIRECT(DT, 256, 256, 64, 2, 4, 4),    \
        TDG_SHAPE(DT, 256, 128, 128, 2, 2), TDG_DIRECT(DT, 256, 128, 128, 2, 2, 3),      \
        TDG_DIRECT_G(DT, 256, 128, 128, 2, 2, 3), TDG_SHAPE(DT, 128, 128, 128, 2, 2),    \
        TDG_DIRECT(DT, 128, 128, 128, 2, 2, 3), TDG_DIRECT(DT, 128, 128, 128, 2, 2, 4),  \
        TDG_DIRECT_G(DT, 128, 128, 128, 2, 2, 3), TDG_DIRECT_G(DT, 128, 128, 128, 2, 2, 4), \
        TDG_SHAPE(DT, 128, 64, 128, 4, 1), TDG_DIRECT(DT, 128, 64, 128, 4, 1, 4),        \
        TDG_DIRECT(DT, 128, 64, 128, 4, 1, 6), TDG_DIRECT_G(DT, 128, 64, 128, 4, 1, 4),  \
        TDG_DIRECT_G(DT, 128, 64, 128, 4, 1, 6), TDG_SHAPE(DT, 64, 64, 128, 2, 2),       \
        TDG_DIRECT(DT, 64, 64, 128, 2, 2, 4), TDG_DIRECT(DT, 64, 64, 128, 2, 2, 8),      \
        TDG_DIRECT_G(DT, 64, 64, 128, 2, 2, 4), TDG_DIRECT_G(DT, 64, 64, 128, 2, 2, 8)

// FP32 inputs: v_mfma_f32_32x32x2_f32 does 8x fewer operations per byte of
// LDS traffic than the FP16 MFMA, so the shapes are the same tiles with fewer
// rings.  The 4-wave 256 x 256 tile is left out: its 256 accumulator
// registers plus four MFMAs per K step per block spill.
#define TDG_SHAPES_F32(DT)                                                                \
    TDG_SHAPE(DT, 256, 256, 128, 2, 4), TDG_SHAPE(DT, 128, 128, 128, 2, 2),              \
        TDG_DIRECT(DT, 128, 128, 128, 2, 2, 3), TDG_DIRECT_G(DT, 128, 128, 128, 2, 2, 3), \
        TDG_SHAPE(DT, 128, 64, 128, 4, 1), TDG_DIRECT(DT, 128, 64, 128, 4, 1, 4),        \
        TDG_DIRECT_G(DT, 128, 64, 128, 4, 1, 4), TDG_SHAPE(DT, 64, 64, 128, 2, 2),       \
        TDG_DIRECT(DT, 64, 64, 128, 2, 2, 4), TDG_DIRECT_G(DT, 64, 64, 128, 2, 2, 4)

// Each dtype's table is its own translation unit (TDG_BUILD_DT = 0, 1 or 2),
// so the three compile in parallel.
#if TDG_BUILD_DT == 0
static const KernelEntry kTable[] = {TDG_SHAPES(DT_F16)};
const KernelEntry *kernel_table_f16(int *count) {
#elif TDG_BUILD_DT == 1
static const KernelEntry kTable[] = {TDG_SHAPES(DT_I8)};
const KernelEntry *kernel_table_i8(int *count) {
#else
static const KernelEntry kTable[] = {TDG_SHAPES_F32(DT_F32)};
const KernelEntry *kernel_table_f32(int *count) {
#endif
    *count = (int)(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace tdg
