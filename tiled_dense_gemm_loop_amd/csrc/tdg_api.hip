// tdg_api.hip -- host side of the C ABI declared in include/tdgemm.h:
// argument validation, the tile/variant planner and kernel dispatch.
//
// Validation and planning are plain host arithmetic and run before any HIP
// call, so a bad argument never reaches the device.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "tdg_internal.h"
#include "tdg_kernels.hpp"
#include "tdgemm.h"

namespace tdg {

// TDG_DEBUG_* bits passed to every GEMM launch (tdg_set_debug_flags).
static std::atomic<int> debug_flags{0};

// The three dtype tables, concatenated once.
const KernelEntry *kernel_table(int *count) {
    static std::vector<KernelEntry> all;
    static std::once_flag once;
    std::call_once(once, [] {
        int nf = 0, ni = 0, n32 = 0;
        const KernelEntry *f = kernel_table_f16(&nf);
        const KernelEntry *i = kernel_table_i8(&ni);
        const KernelEntry *w = kernel_table_f32(&n32);
        all.insert(all.end(), f, f + nf);
        all.insert(all.end(), i, i + ni);
        all.insert(all.end(), w, w + n32);
    });
    *count = (int)all.size();
    return all.data();
}

// Whether the current device is gfx950 (cached per device).
static std::mutex g_dev_mutex;
static signed char g_dev_ok[64];  // 0 unknown, 1 gfx950, -1 other

int device_check() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TDG_ERR_NO_DEVICE;
    if (dev < 0 || dev >= 64) return TDG_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TDG_ERR_NO_DEVICE;
        g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return g_dev_ok[dev] == 1 ? TDG_OK : TDG_ERR_NO_DEVICE;
}

}  // namespace tdg

namespace {

using tdg::KernelEntry;
using tdg::device_check;

constexpr int kNumCU = 256;               // MI355X compute units
constexpr int kLdsPerCU = 160 * 1024;     // gfx950 LDS per CU
constexpr int kWaveSlotsPerCU = 4 * 8;    // 4 SIMDs x 8 wave slots
constexpr int kRegsPerLanePerSIMD = 512;  // unified VGPR + AGPR file

int elem_size(int dtype) {
    return dtype == TDG_DTYPE_F16F32 ? 2 : (dtype == TDG_DTYPE_I8I32 ? 1 : 4);
}

// Largest M, N or K: the kernels index rows, columns and k in 32 bits and
// form sums such as (tile start + tile extent) on them, so every size keeps a
// margin of 2^16 below 2^31.
constexpr int64_t kMaxDim = ((int64_t)1 << 31) - ((int64_t)1 << 16);

bool dims_ok(int64_t M, int64_t N, int64_t K) {
    return M >= 0 && N >= 0 && K >= 0 && M <= kMaxDim && N <= kMaxDim && K <= kMaxDim;
}

bool dtype_ok(int dtype) {
    return dtype == TDG_DTYPE_F16F32 || dtype == TDG_DTYPE_I8I32 || dtype == TDG_DTYPE_F32F32;
}

// ---------------------------------------------------------------- validation

bool ranges_overlap(uintptr_t a0, uint64_t alen, uintptr_t b0, uint64_t blen) {
    if (alen == 0 || blen == 0) return false;
    return a0 < b0 + blen && b0 < a0 + alen;
}

// Whether rows x ld elements of es bytes fit in int64 (every matrix that can
// exist does; a larger leading dimension is rejected before any arithmetic
// on it could overflow).
bool extent_ok(int64_t rows, int64_t ld, int es) {
    return rows == 0 || ld <= INT64_MAX / es / rows;
}

// Bytes spanned by a rows x cols row-major matrix with leading dimension ld
// (cols <= ld and extent_ok hold).
uint64_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int es) {
    if (rows == 0 || cols == 0) return 0;
    return (uint64_t)((rows - 1) * ld + cols) * (uint64_t)es;
}

int validate(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
             int64_t ldb, const void *C, int64_t ldc) {
    if (!dtype_ok(dtype)) return TDG_ERR_INVALID_ARG;
    if (!dims_ok(M, N, K)) return TDG_ERR_INVALID_ARG;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return TDG_ERR_INVALID_ARG;
    if (M > 0 && K > 0 && !A) return TDG_ERR_INVALID_ARG;
    if (K > 0 && N > 0 && !B) return TDG_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && !C) return TDG_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    if (!extent_ok(M, lda, es) || !extent_ok(K, ldb, es) || !extent_ok(M, ldc, 4))
        return TDG_ERR_INVALID_ARG;
    const uint64_t cspan = span_bytes(M, N, ldc, 4);
    if (ranges_overlap((uintptr_t)C, cspan, (uintptr_t)A, span_bytes(M, K, lda, es)) ||
        ranges_overlap((uintptr_t)C, cspan, (uintptr_t)B, span_bytes(K, N, ldb, es)))
        return TDG_ERR_INVALID_ARG;
    return TDG_OK;
}

// ------------------------------------------------------------------ planner

int cfg_waves(const KernelEntry &e) { return e.wm * e.wn; }
int cfg_bk(const KernelEntry &e) { return e.bkb / elem_size(e.dtype); }

bool same_tile(const KernelEntry &a, const KernelEntry &b) {
    return a.dtype == b.dtype && a.bm == b.bm && a.bn == b.bn && a.bkb == b.bkb && a.wm == b.wm &&
           a.wn == b.wn;
}

// Does this request (zeros = "any") match the entry's tile shape?
bool tile_matches(const tdg_config &req, const KernelEntry &e) {
    return (req.bm == 0 || req.bm == e.bm) && (req.bn == 0 || req.bn == e.bn) &&
           (req.bk == 0 || req.bk == cfg_bk(e)) && (req.waves == 0 || req.waves == cfg_waves(e));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Whether the unguarded fast path may run: whole tiles, 16-byte aligned
// operands and rows, and per-tile offsets inside 32 bits.
// A shape of whole tiles: M, N and K multiples of the tile, so every row
// of a K tile is whole 16-byte chunks and no chunk runs past its row.  The
// unchecked direct-to-LDS loop serves it at any alignment: the LDS DMA reads
// its 16 bytes from any byte address (the parity tests run it at every
// byte offset of a chunk).  The unchecked register and sequential loops load through 16-byte
// vector types and also need 16-byte aligned rows (aligned_operands).
bool fast_ok(const KernelEntry &e, int64_t M, int64_t N, int64_t K) {
    const int bk = cfg_bk(e);
    return K > 0 && M % e.bm == 0 && N % e.bn == 0 && K % bk == 0;
}

// Whether the chunk that holds an operand's last byte (rows x cols elements
// of es bytes, leading dimension ld) reaches into another 4 KiB page.
// Chunks sit on a 16-byte grid from each row's first byte, so that chunk
// starts at the last row's first byte plus the last byte's offset rounded
// down to 16.  With 16-byte aligned rows it never does.
bool end_chunk_crosses_page(const void *base, int64_t rows, int64_t ld, int64_t cols, int es) {
    if (rows <= 0 || cols <= 0) return false;
    const uintptr_t row = (uintptr_t)base + (uintptr_t)((rows - 1) * ld * es);
    const uintptr_t last = row + (uintptr_t)(cols * es - 1);             // the last byte
    const uintptr_t start = row + ((uintptr_t)(cols * es - 1) & ~(uintptr_t)15);
    return ((start + 15) >> 12) != (last >> 12);
}

// The bounds-checked direct-to-LDS loop runs ragged shapes at any
// alignment: chunks that start outside an operand are fetched from a zero
// block and those that start inside are fetched whole; the kernel clears
// A's bytes at k >= K when K splits a chunk (B's bytes past N feed only C
// columns that are not stored).  A chunk read whole can run past the
// operand's end only at the end of its last row, and must not enter a page
// that holds no byte of the operand (such a page need not be mapped):
// whether both operands' last chunks stay in their pages.  Operands placed
// otherwise are left to the bounds-checked register loop, whose loads stay
// in the page of their first byte.
bool ends_in_page(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                  int64_t ldb) {
    const int es = elem_size(dtype);
    return !end_chunk_crosses_page(A, M, lda, K, es) && !end_chunk_crosses_page(B, K, ldb, N, es);
}

bool aligned_operands(int dtype, const void *A, int64_t lda, const void *B, int64_t ldb) {
    const int es = elem_size(dtype);
    return ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0) && ((lda * es) % 16 == 0) &&
           ((ldb * es) % 16 == 0);
}

// Whether the per-lane 32-bit offsets of a kernel reach every chunk it loads
// from A and B.  A thread's first chunk sits (NT / CPR - 1) rows below the
// tile's first row at most (NT threads, CPR 16-byte chunks per image row:
// 127 rows for the 8-wave 256-wide tiles with a 64-byte K tile), and the
// offset adds at most one row's worth of chunk bytes; the hardware reads the
// offset as an unsigned 32-bit value added to a 64-bit base.  Later chunks
// and K tiles move the wave-uniform 64-bit base, not the offset.
bool offsets_fit(const KernelEntry &e, int64_t lda, int64_t ldb) {
    const uint64_t es = (uint64_t)elem_size(e.dtype);
    const uint64_t nt = (uint64_t)cfg_waves(e) * 64u;
    const uint64_t a_cpr = (uint64_t)e.bkb / 16u, b_cpr = (uint64_t)e.bn * es / 16u;
    const uint64_t a_rows = nt / a_cpr, b_rows = nt / b_cpr;
    const uint64_t lim = 0xFFFFFFFFull;
    auto fits = [&](uint64_t rows, int64_t ld, uint64_t row_bytes) {
        if (ld < 0) return false;
        if (rows <= 1) return row_bytes <= lim;
        const uint64_t ld_bytes = (uint64_t)ld * es;  // extent_ok bounds ld * es
        return ld_bytes <= (lim - row_bytes) / (rows - 1);
    };
    return fits(a_rows, lda, (uint64_t)e.bkb) && fits(b_rows, ldb, (uint64_t)e.bn * es);
}

// Largest tile side (bm, bn, bk) the tile arithmetic accepts: far beyond any
// tile that fits the LDS, and small enough for its products to stay exact.
constexpr int kMaxTileSide = 1 << 16;

// Estimated 32-bit registers per lane: accumulators, register staging of one
// K tile (not for direct-to-LDS) and two sets of MFMA fragments.  (64-bit
// arithmetic: tiles up to kMaxTileSide on a side.)
int est_regs(int bm, int bn, int bkb, int waves, int variant) {
    const int64_t lanes = (int64_t)waves * 64;
    const int64_t acc = (int64_t)bm * bn / lanes;
    const int64_t staging = variant == TDG_VARIANT_DIRECT_LDS ? 0 : ((int64_t)bm + bn) * bkb / lanes / 4;
    // a wave owns about (bm * bn / waves) outputs, split into 32x32 blocks
    const double wave_side = 32.0 * __builtin_sqrt((double)bm * bn / waves / 1024.0);
    const int64_t frags = 2 * 2 * 4 * (int64_t)(wave_side / 32.0 + 0.5);
    const int64_t total = acc + staging + frags + 24;
    return total > INT32_MAX ? INT32_MAX : (int)total;
}

// Whether tile rows walk K from their own offsets: when all of B fits in half
// an XCD's 4 MB L2, B is served from L2 in any order, and rotating the walk
// spreads A's concurrent HBM reads over the channels.
bool k_rotation(int dtype, int64_t N, int64_t K) {
    return (double)K * (double)N * elem_size(dtype) <= (double)(2 << 20);
}

// The pages' planning arithmetic for one tile and problem.
void tile_figures(int dtype, int bm, int bn, int bk, int waves, int stages, int variant, int64_t M,
                  int64_t N, int64_t K, tdg_plan_info *info) {
    const int es = elem_size(dtype);
    // "Pipeline GPU Kernel", Step 2: operations per byte loaded per tile.
    const double flops = 2.0 * bm * bn * bk;
    const double bytes = ((double)bm * bk + (double)bk * bn) * es;
    info->ratio = flops / bytes;
    info->band = info->ratio < 5.0 ? 0 : (info->ratio <= 20.0 ? 1 : 2);
    // "Pipeline GPU Kernel", Step 1: one buffer = (BM*BK + BK*BN)*sizeof(T).
    info->lds_bytes = (size_t)stages * ((size_t)bm * bk + (size_t)bk * bn) * (size_t)es;
    const int by_lds = info->lds_bytes ? (int)(kLdsPerCU / info->lds_bytes) : 64;
    const int by_waves = kWaveSlotsPerCU / waves;
    const int regs = est_regs(bm, bn, bk * es, waves, variant);
    int waves_per_simd = kRegsPerLanePerSIMD / (regs < 1 ? 1 : regs);
    if (waves_per_simd > 8) waves_per_simd = 8;
    const int by_regs = waves_per_simd * 4 / waves;
    int wg = by_lds < by_waves ? by_lds : by_waves;
    info->wg_per_cu = wg < by_regs ? wg : by_regs;
    info->num_tiles = ceil_div(K, bk);
    info->grid = ceil_div(M, bm) * ceil_div(N, bn);
    info->est_regs = regs;
    info->guarded = 0;
    // MI355X MFMA operations per clock per CU (dense peak / 256 CUs / 2.4 GHz)
    const double ops_per_clk = dtype == TDG_DTYPE_F16F32 ? 4096.0
                               : dtype == TDG_DTYPE_I8I32 ? 8192.0
                                                          : 256.0;
    info->need_bytes_per_clk = ops_per_clk / info->ratio;
    // one 32x32 MFMA covers k = 16 (FP16), 32 (INT8) or 2 (FP32)
    const double k_mfma = dtype == TDG_DTYPE_F16F32 ? 16.0 : dtype == TDG_DTYPE_I8I32 ? 32.0 : 2.0;
    const double mfmas = (double)bm * bn * bk / (32.0 * 32.0 * k_mfma);
    const double loads = bytes / 1024.0;  // 64 lanes x 16 bytes per wave instruction
    info->mfma_per_load = mfmas / loads;
    info->pipelined = variant != TDG_VARIANT_SINGLE && info->num_tiles >= 2;
    info->k_rotated = k_rotation(dtype, N, K) ? 1 : 0;
}

void fill_info(const KernelEntry &e, int variant, int stages, int64_t M, int64_t N, int64_t K,
               bool guarded, tdg_plan_info *info) {
    if (!info) return;
    tile_figures(e.dtype, e.bm, e.bn, cfg_bk(e), cfg_waves(e), stages, variant, M, N, K, info);
    info->guarded = guarded ? 1 : 0;
}

// Measured kernel time of every built direct-to-LDS configuration with a
// 128-byte K tile, as a function of the number of workgroups n and of K:
// T(n, K) = a + b * K microseconds, interpolated between the n of kPerfN.
// Measured on one MI355X at K = 1024 and K = 4096 with the tiles laid out
// close to square, FP16 and INT8 as HIP-graph replays, FP32 as back-to-back
// launches; each series is non-decreasing in n (tune_planner.py in the
// package measures and prints this table).  The rows of a dtype are in
// preference order for near ties.
struct PerfRow {
    int dtype, bm, bn, waves, stages;
    float a[12], b[12];
};
const int kPerfN[12] = {32, 64, 128, 192, 256, 320, 384, 512, 768, 1024, 1536, 2304};
const PerfRow kPerf[] = {
    {0, 256, 256, 8, 2, {6.77f, 6.29f, 6.54f, 9.68f, 13.94f, 18.70f, 18.39f, 23.92f, 33.90f, 41.53f, 57.69f, 84.83f},
     {0.015843f, 0.016309f, 0.018265f, 0.021527f, 0.024521f, 0.039971f, 0.042311f, 0.048005f, 0.071582f, 0.095768f, 0.144336f, 0.216790f}},
    {0, 256, 256, 4, 2, {6.22f, 8.06f, 10.61f, 12.78f, 16.02f, 20.70f, 21.60f, 26.80f, 36.89f, 45.68f, 62.36f, 92.92f},
     {0.018724f, 0.018278f, 0.019157f, 0.022106f, 0.025075f, 0.042393f, 0.043271f, 0.048988f, 0.073167f, 0.097637f, 0.148610f, 0.221341f}},
    {0, 256, 128, 4, 2, {3.17f, 3.17f, 4.05f, 6.29f, 7.77f, 9.70f, 9.71f, 12.76f, 19.56f, 23.27f, 33.60f, 53.08f},
     {0.012070f, 0.012070f, 0.012207f, 0.012708f, 0.014417f, 0.025837f, 0.026351f, 0.028906f, 0.042588f, 0.058900f, 0.087894f, 0.130293f}},
    {0, 256, 128, 4, 3, {4.70f, 4.35f, 4.51f, 5.89f, 7.79f, 11.67f, 10.76f, 13.71f, 18.86f, 22.03f, 35.12f, 56.21f},
     {0.011686f, 0.012028f, 0.012594f, 0.013633f, 0.015039f, 0.025820f, 0.026803f, 0.029248f, 0.044447f, 0.061670f, 0.090225f, 0.133105f}},
    {0, 128, 128, 4, 4, {4.13f, 3.83f, 3.70f, 4.40f, 4.79f, 7.24f, 7.12f, 6.92f, 10.00f, 12.14f, 18.23f, 29.88f},
     {0.006149f, 0.006442f, 0.006849f, 0.007142f, 0.008298f, 0.014173f, 0.014284f, 0.016413f, 0.024785f, 0.033926f, 0.051003f, 0.074248f}},
    {0, 128, 128, 4, 2, {-0.17f, -0.17f, -0.43f, 2.96f, 3.32f, 4.75f, 4.00f, 5.62f, 8.58f, 10.81f, 14.00f, 22.82f},
     {0.010033f, 0.010033f, 0.010280f, 0.009811f, 0.010462f, 0.011647f, 0.013223f, 0.015072f, 0.023958f, 0.029417f, 0.044141f, 0.066022f}},
    {0, 128, 128, 4, 3, {3.94f, 3.94f, 3.80f, 4.28f, 5.18f, 7.51f, 6.97f, 6.27f, 9.67f, 13.23f, 20.39f, 25.15f},
     {0.007936f, 0.007936f, 0.008203f, 0.008643f, 0.009186f, 0.016755f, 0.017285f, 0.019479f, 0.029170f, 0.038005f, 0.055957f, 0.087878f}},
    {0, 128, 64, 4, 4, {3.08f, 3.08f, 2.88f, 3.07f, 3.22f, 5.03f, 5.03f, 5.48f, 5.10f, 9.90f, 13.58f, 17.33f},
     {0.005107f, 0.005107f, 0.005371f, 0.005492f, 0.005726f, 0.010423f, 0.010423f, 0.010911f, 0.017835f, 0.022386f, 0.033701f, 0.050964f}},
    {0, 128, 64, 4, 2, {-0.86f, -1.04f, -1.27f, -0.19f, -0.53f, 1.85f, 2.14f, 4.13f, 4.03f, 6.81f, 6.98f, 8.02f},
     {0.008848f, 0.009027f, 0.009339f, 0.009245f, 0.009583f, 0.009395f, 0.009323f, 0.009808f, 0.015495f, 0.021530f, 0.029329f, 0.044303f}},
    {0, 128, 64, 4, 6, {3.70f, 3.70f, 3.76f, 3.97f, 4.00f, 6.69f, 6.69f, 6.81f, 8.60f, 12.69f, 17.86f, 23.08f},
     {0.006006f, 0.006006f, 0.006110f, 0.006348f, 0.006689f, 0.012233f, 0.012233f, 0.013005f, 0.019616f, 0.025550f, 0.037985f, 0.057363f}},
    {0, 64, 64, 4, 4, {2.89f, 2.89f, 2.89f, 3.03f, 3.15f, 1.25f, 1.36f, 1.40f, 4.49f, 4.46f, 6.03f, 7.97f},
     {0.003490f, 0.003490f, 0.003555f, 0.003581f, 0.003682f, 0.007002f, 0.006976f, 0.007884f, 0.010915f, 0.013770f, 0.019769f, 0.028906f}},
    {0, 64, 64, 4, 2, {-1.20f, -1.20f, -1.29f, -1.17f, -1.31f, 0.31f, 0.41f, 2.20f, 3.17f, 4.01f, 5.04f, 6.68f},
     {0.007660f, 0.007660f, 0.007790f, 0.007965f, 0.008252f, 0.007946f, 0.007923f, 0.007855f, 0.010518f, 0.013734f, 0.018910f, 0.028861f}},
    {0, 64, 64, 4, 8, {3.45f, 3.45f, 3.46f, 3.50f, 3.52f, 5.31f, 5.43f, 5.57f, 7.18f, 9.51f, 12.85f, 17.71f},
     {0.003353f, 0.003353f, 0.003408f, 0.003548f, 0.003623f, 0.006868f, 0.006839f, 0.007028f, 0.011003f, 0.014186f, 0.021520f, 0.032646f}},
    {1, 256, 256, 8, 2, {6.69f, 6.69f, 7.87f, 10.51f, 13.65f, 18.41f, 18.68f, 24.17f, 34.51f, 41.58f, 59.17f, 84.37f},
     {0.007848f, 0.007848f, 0.008480f, 0.010150f, 0.012184f, 0.019854f, 0.020993f, 0.023818f, 0.035036f, 0.047500f, 0.071198f, 0.108330f}},
    {1, 256, 256, 4, 2, {6.71f, 7.25f, 9.36f, 12.47f, 15.77f, 20.82f, 21.89f, 26.63f, 36.92f, 45.14f, 63.53f, 93.19f},
     {0.009320f, 0.009294f, 0.009756f, 0.010752f, 0.012409f, 0.020918f, 0.021250f, 0.024095f, 0.035811f, 0.047829f, 0.072070f, 0.110345f}},
    {1, 256, 128, 4, 2, {3.81f, 3.81f, 4.55f, 6.14f, 7.98f, 10.22f, 9.84f, 12.17f, 17.77f, 21.86f, 30.96f, 48.23f},
     {0.006250f, 0.006250f, 0.006139f, 0.006410f, 0.007308f, 0.013161f, 0.013538f, 0.014642f, 0.021921f, 0.029548f, 0.044447f, 0.067640f}},
    {1, 256, 128, 4, 3, {4.98f, 4.98f, 5.69f, 7.01f, 8.34f, 11.78f, 11.65f, 14.02f, 19.37f, 24.69f, 34.99f, 49.28f},
     {0.005794f, 0.005794f, 0.005788f, 0.006344f, 0.007321f, 0.012816f, 0.013079f, 0.014323f, 0.021758f, 0.029580f, 0.045208f, 0.068698f}},
    {1, 128, 128, 4, 4, {4.24f, 4.24f, 4.29f, 4.79f, 5.41f, 8.12f, 8.48f, 8.56f, 12.01f, 14.95f, 20.73f, 31.20f},
     {0.003236f, 0.003236f, 0.003340f, 0.003584f, 0.004176f, 0.007279f, 0.007191f, 0.007887f, 0.012035f, 0.016507f, 0.025661f, 0.038483f}},
    {1, 128, 128, 4, 2, {2.92f, 2.92f, 2.24f, 2.98f, 3.91f, 4.50f, 4.50f, 5.94f, 8.51f, 11.44f, 16.29f, 21.57f},
     {0.004336f, 0.004336f, 0.005000f, 0.005098f, 0.005286f, 0.006807f, 0.006807f, 0.007454f, 0.012572f, 0.014378f, 0.021429f, 0.033288f}},
    {1, 128, 128, 4, 3, {4.00f, 4.00f, 4.02f, 4.68f, 5.59f, 7.65f, 7.92f, 8.37f, 11.99f, 14.12f, 19.94f, 29.37f},
     {0.003968f, 0.003968f, 0.004063f, 0.004121f, 0.004411f, 0.008350f, 0.008285f, 0.008763f, 0.014046f, 0.018988f, 0.028105f, 0.041693f}},
    {1, 128, 64, 4, 4, {3.37f, 3.37f, 3.45f, 3.25f, 3.56f, 5.26f, 4.80f, 5.83f, 7.17f, 9.57f, 15.75f, 19.49f},
     {0.002572f, 0.002572f, 0.002552f, 0.003018f, 0.002985f, 0.005339f, 0.005827f, 0.005664f, 0.008796f, 0.011924f, 0.017139f, 0.026686f}},
    {1, 128, 64, 4, 2, {2.34f, 2.34f, 2.26f, 1.99f, 1.72f, 2.99f, 2.56f, 4.12f, 3.92f, 5.61f, 8.09f, 7.92f},
     {0.003958f, 0.003958f, 0.004040f, 0.004704f, 0.005068f, 0.005000f, 0.005723f, 0.005882f, 0.008750f, 0.012041f, 0.016445f, 0.025176f}},
    {1, 128, 64, 4, 6, {3.67f, 3.67f, 3.84f, 4.02f, 4.29f, 6.15f, 6.28f, 7.60f, 9.56f, 12.37f, 20.80f, 26.84f},
     {0.003210f, 0.003210f, 0.003193f, 0.003314f, 0.003447f, 0.006582f, 0.006549f, 0.006413f, 0.009932f, 0.013389f, 0.018991f, 0.029076f}},
    {1, 64, 64, 4, 4, {2.92f, 2.92f, 2.92f, 2.59f, 2.71f, 2.82f, 2.87f, 3.00f, 3.61f, 4.10f, 7.34f, 8.01f},
     {0.001790f, 0.001790f, 0.001790f, 0.002246f, 0.002233f, 0.003568f, 0.003880f, 0.004307f, 0.006429f, 0.008646f, 0.011940f, 0.017878f}},
    {1, 64, 64, 4, 2, {2.86f, 2.84f, 2.77f, 1.34f, 1.58f, 2.14f, 1.80f, 2.41f, 1.87f, 3.60f, 4.81f, 5.07f},
     {0.001979f, 0.001999f, 0.002204f, 0.003851f, 0.003851f, 0.003997f, 0.004518f, 0.004600f, 0.006855f, 0.008327f, 0.011286f, 0.017695f}},
    {1, 64, 64, 4, 8, {3.36f, 3.36f, 3.34f, 3.56f, 3.55f, 5.10f, 4.70f, 5.28f, 7.12f, 9.50f, 14.80f, 21.06f},
     {0.001868f, 0.001868f, 0.001914f, 0.002194f, 0.002204f, 0.003835f, 0.004574f, 0.004469f, 0.006768f, 0.008763f, 0.012832f, 0.018688f}},
    {2, 256, 256, 8, 2, {10.57f, 9.31f, 11.91f, 20.51f, 30.15f, 20.15f, 19.50f, 30.60f, 28.52f, 37.24f, 58.85f, 81.72f},
     {0.218822f, 0.220052f, 0.220804f, 0.218704f, 0.217191f, 0.435628f, 0.436260f, 0.438535f, 0.662718f, 0.882604f, 1.319268f, 1.980283f}},
    {2, 128, 128, 4, 2, {5.57f, 5.78f, 5.47f, 3.07f, 3.36f, 7.70f, 7.70f, 4.88f, -0.56f, 12.36f, 18.32f, -53.73f},
     {0.057122f, 0.057070f, 0.057803f, 0.061064f, 0.063021f, 0.111924f, 0.111924f, 0.116875f, 0.183105f, 0.225020f, 0.338024f, 0.580762f}},
    {2, 128, 128, 4, 3, {5.35f, 5.55f, 4.86f, 2.67f, 3.59f, 9.95f, 9.95f, 7.59f, 11.57f, 12.28f, 20.84f, 23.93f},
     {0.057891f, 0.057842f, 0.058584f, 0.061829f, 0.062998f, 0.117360f, 0.117360f, 0.121416f, 0.179684f, 0.239844f, 0.357780f, 0.537057f}},
    {2, 128, 64, 4, 4, {5.65f, 5.65f, 5.53f, 4.60f, 4.05f, 7.46f, 7.46f, 6.98f, 9.94f, 13.54f, 13.88f, 20.59f},
     {0.030182f, 0.030182f, 0.030306f, 0.031214f, 0.032650f, 0.061992f, 0.061992f, 0.063454f, 0.094049f, 0.123522f, 0.187900f, 0.281540f}},
    {2, 128, 64, 4, 2, {4.95f, 4.95f, 4.93f, 4.50f, 3.95f, 6.19f, 6.50f, 7.73f, 3.93f, 26.93f, 11.16f, 19.12f},
     {0.030426f, 0.030426f, 0.030560f, 0.031615f, 0.033219f, 0.058350f, 0.058275f, 0.058675f, 0.090186f, 0.120094f, 0.172370f, 0.254694f}},
    {2, 64, 64, 4, 4, {3.67f, 3.67f, 3.62f, 4.13f, 4.45f, 3.83f, 3.78f, 4.43f, 6.00f, 5.38f, 1.14f, 10.07f},
     {0.016243f, 0.016243f, 0.016289f, 0.016517f, 0.016693f, 0.030179f, 0.030225f, 0.030381f, 0.059847f, 0.060563f, 0.095456f, 0.151530f}},
    {2, 64, 64, 4, 2, {3.91f, 3.91f, 3.73f, 3.63f, 4.46f, 4.69f, 4.97f, 4.68f, 4.27f, 2.28f, 5.06f, 8.20f},
     {0.016169f, 0.016169f, 0.016351f, 0.016449f, 0.016914f, 0.029860f, 0.029792f, 0.030332f, 0.045706f, 0.062083f, 0.103734f, 0.145026f}},
};

// Interpolated T(x, K) of one row; below the first n the time is flat, and
// K below 1024 is taken as 1024 (small products sit at the launch floor,
// where the line through the two measured K says nothing).  The measured
// points are first made non-decreasing in n at this K (a running maximum:
// more workgroups never finish sooner) and at least kMinUs (no launch is
// free), so the model is positive and non-decreasing in n and, with every
// slope b >= 0, in K, whatever the fitted lines do between and beyond the
// two measured K.
constexpr double kMinUs = 1.0;
double perf_at(const PerfRow &r, int64_t x, int64_t K) {
    const double k = (double)(K < 1024 ? 1024 : K);
    constexpr int P = (int)(sizeof(kPerfN) / sizeof(kPerfN[0]));
    double t[P];
    double run = kMinUs;
    for (int i = 0; i < P; i++) {
        const double v = (double)r.a[i] + (double)(r.b[i] > 0.0f ? r.b[i] : 0.0f) * k;
        run = v > run ? v : run;
        t[i] = run;
    }
    if (x <= kPerfN[0]) return t[0];
    for (int i = 1; i < P; i++) {
        if (x <= kPerfN[i]) {
            const double f = (double)(x - kPerfN[i - 1]) / (double)(kPerfN[i] - kPerfN[i - 1]);
            return t[i - 1] + f * (t[i] - t[i - 1]);
        }
    }
    return t[P - 1] * (double)x / (double)kPerfN[P - 1];
}

// Predicted kernel time for `tiles` workgroups: full rounds of slots =
// 256 CUs x workgroups per CU, then the last, partial round.
double predict_us(const PerfRow &r, int wg_per_cu, int64_t tiles, int64_t K) {
    const int64_t slots = (int64_t)kNumCU * (wg_per_cu > 0 ? wg_per_cu : 1);
    const int64_t full = (tiles - 1) / slots;
    const int64_t rem = tiles - full * slots;
    return (double)full * perf_at(r, slots, K) + perf_at(r, rem, K);
}

// The SINGLE-variant table entry that names a tile shape (tile, waves).
const KernelEntry *tile_entry(int dtype, int bm, int bn, int bkb, int waves) {
    int count = 0;
    const KernelEntry *table = tdg::kernel_table(&count);
    for (int i = 0; i < count; i++) {
        const KernelEntry &e = table[i];
        if (e.dtype == dtype && !e.guard && e.variant == TDG_VARIANT_SINGLE && e.bm == bm &&
            e.bn == bn && e.bkb == bkb && cfg_waves(e) == waves)
            return &e;
    }
    return nullptr;
}

struct Choice {
    const KernelEntry *tile;  // tile shape (its SINGLE entry)
    int stages;               // ring depth for the direct-to-LDS loop; 0 = none measured
};

// The table's times are for 16-byte aligned rows.  With rows off that grid
// a 128-byte K-tile row of A spans two 128-byte lines instead of one, and
// the copy of every tile costs more, the more so the more bytes a
// configuration copies per compute unit and the shallower its ring.
// Measured at 4096^3 (rows 2 bytes off, every direct-to-LDS configuration):
// about 7 (FP16) to 10 (INT8) us per MB of L2 -> LDS traffic per compute
// unit with two buffers, and about three quarters of that with three or
// four (256 x 128: 45 against 33 us; 128 x 128: 59 against 46 us, FP16).
constexpr double kMisalignedUsPerMB = 8.0;

double misaligned_penalty_us(int64_t grid, int bm, int bn, int stages, int64_t K, int es) {
    const double mb_per_cu = (double)grid * (bm + bn) * (double)K * es / kNumCU / 1e6;
    return kMisalignedUsPerMB * mb_per_cu * (stages > 2 ? 0.75 : 1.0);
}

// Tile shape, waves and ring depth for a product: the measured configuration
// with the least predicted time (a near tie, within 3%, goes to the earlier
// row), with the copy's extra cost added when the rows are not 16-byte
// aligned.  Requests outside the measured table (other K tiles, or a tile,
// wave count or ring depth no row has) fall back to the largest tile that
// gives every compute unit a workgroup, or the one giving the most.
Choice choose_config(int dtype, int64_t M, int64_t N, int64_t K, const tdg_config &req,
                     bool rows_aligned = true) {
    const PerfRow *best = nullptr;
    const KernelEntry *best_tile = nullptr;
    double best_t = 0.0;
    const int es = elem_size(dtype);
    const bool any_variant_ok = req.variant == TDG_VARIANT_AUTO || req.variant == TDG_VARIANT_DIRECT_LDS;
    if (req.bk == 0 || (int64_t)req.bk * es == 128) {
        for (const PerfRow &r : kPerf) {
            if (r.dtype != dtype) continue;
            if ((req.bm && req.bm != r.bm) || (req.bn && req.bn != r.bn) ||
                (req.waves && req.waves != r.waves))
                continue;
            if (req.lds_stages && any_variant_ok && req.lds_stages != r.stages) continue;
            const KernelEntry *t = tile_entry(dtype, r.bm, r.bn, 128, r.waves);
            if (!t) continue;
            tdg_plan_info fig;
            tile_figures(dtype, r.bm, r.bn, 128 / es, r.waves, r.stages, TDG_VARIANT_DIRECT_LDS, M, N,
                         K, &fig);
            double t_us = predict_us(r, fig.wg_per_cu, fig.grid, K);
            if (!rows_aligned) t_us += misaligned_penalty_us(fig.grid, r.bm, r.bn, r.stages, K, es);
            if (!best || t_us < best_t * 0.97) {
                best = &r;
                best_tile = t;
                best_t = t_us;
            }
        }
    }
    if (best) return Choice{best_tile, best->stages};

    int count = 0;
    const KernelEntry *table = tdg::kernel_table(&count);
    const KernelEntry *pick = nullptr;
    int64_t best_area = -1, best_grid = -1;
    bool best_fills = false;
    for (int i = 0; i < count; i++) {
        const KernelEntry &e = table[i];
        if (e.dtype != dtype || e.guard || e.variant != TDG_VARIANT_SINGLE) continue;
        if (!tile_matches(req, e)) continue;
        if (req.bk == 0 && e.bkb != 128) continue;
        const int64_t grid = ceil_div(M, e.bm) * ceil_div(N, e.bn);
        const int64_t area = (int64_t)e.bm * e.bn;
        const bool fills = grid >= kNumCU;
        bool better;
        if (!pick) better = true;
        else if (fills != best_fills) better = fills;
        else if (fills) better = area > best_area;
        else better = grid > best_grid || (grid == best_grid && area > best_area);
        if (better) {
            pick = &e;
            best_area = area;
            best_grid = grid;
            best_fills = fills;
        }
    }
    return Choice{pick, 0};
}

const KernelEntry *find_entry(const KernelEntry &tile, int stages, int variant, bool guard) {
    int count = 0;
    const KernelEntry *table = tdg::kernel_table(&count);
    for (int i = 0; i < count; i++) {
        const KernelEntry &e = table[i];
        if (same_tile(e, tile) && e.stages == stages && e.variant == variant && e.guard == guard)
            return &e;
    }
    return nullptr;
}

struct Resolved {
    const KernelEntry *entry;  // kernel to launch
    int variant, stages;
    bool guarded;
};

// Complete a (possibly partial) request into a runnable kernel.
// `end_ok`: the operands' last chunks stay in their pages (ends_in_page).
int resolve(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
            int64_t ldb, bool end_ok, const tdg_config &req_in, bool pipelined_default, Resolved *out,
            tdg_config *cfg_out, tdg_plan_info *info) {
    tdg_config req = req_in;
    if (req.variant < 0 || req.variant > TDG_VARIANT_DIRECT_LDS) return TDG_ERR_INVALID_ARG;
    if (req.lds_stages < 0 || req.lds_stages > 8) return TDG_ERR_UNSUPPORTED;
    const bool vec_ok = aligned_operands(dtype, A, lda, B, ldb);
    const Choice choice = choose_config(dtype, M, N, K, req, vec_ok);
    const KernelEntry *tile = choice.tile;
    if (!tile) return TDG_ERR_UNSUPPORTED;
    // Ring depth of the direct-to-LDS loop when the caller leaves it open:
    // the chosen configuration's, when it is built in the form asked for
    // (plain or bounds-checked), else two buffers.
    auto direct_stages = [&](bool guarded) {
        if (choice.stages && find_entry(*tile, choice.stages, TDG_VARIANT_DIRECT_LDS, guarded))
            return choice.stages;
        return 2;
    };
    const bool whole = fast_ok(*tile, M, N, K);
    const bool edge = !whole && K > 0 && end_ok;

    int variant = req.variant;
    // With one K tile there is nothing to overlap ("Pipeline GPU Kernel",
    // Step 1: pipelining needs at least two tiles); the planner then runs
    // the sequential form, which computes the same result.
    const bool one_tile = ceil_div(K, cfg_bk(*tile)) < 2;
    if (variant == TDG_VARIANT_AUTO)
        variant = pipelined_default && !one_tile
                      ? (whole || edge ? TDG_VARIANT_DIRECT_LDS : TDG_VARIANT_REG_PREFETCH)
                      : TDG_VARIANT_SINGLE;
    int stages = req.lds_stages;
    if (stages == 0)
        stages = variant == TDG_VARIANT_SINGLE ? 1
                 : variant == TDG_VARIANT_REG_PREFETCH ? 2
                                                       : direct_stages(!whole);
    if (variant == TDG_VARIANT_SINGLE && stages != 1) return TDG_ERR_UNSUPPORTED;
    if (variant == TDG_VARIANT_REG_PREFETCH && stages > 2) return TDG_ERR_UNSUPPORTED;
    if (variant == TDG_VARIANT_DIRECT_LDS && stages < 2) return TDG_ERR_UNSUPPORTED;

    // The direct-to-LDS loop runs unchecked on whole tiles at any alignment;
    // the register and sequential loops only when the rows are also aligned.
    bool guard = variant == TDG_VARIANT_DIRECT_LDS ? !whole : !(whole && vec_ok);
    const KernelEntry *e = nullptr;
    if (!guard) {
        e = find_entry(*tile, stages, variant, false);
    } else if (variant == TDG_VARIANT_DIRECT_LDS) {
        // The DMA needs a valid source for every 16-byte chunk ("Pipeline
        // GPU Kernel", Common Pitfalls): ragged shapes keep the copy in the
        // DMA's bounds-checked form (at the asked ring depth if built, else
        // the tile's preferred one, else two buffers); a K of zero, or an
        // operand whose last chunk would enter a page beyond it (not
        // ends_in_page), runs the bounds-checked register-prefetch loop.
        if (edge) {
            e = find_entry(*tile, stages, variant, true);
            if (!e) {
                stages = direct_stages(true);
                e = find_entry(*tile, stages, variant, true);
            }
            if (!e) {
                stages = 2;
                e = find_entry(*tile, stages, variant, true);
            }
        }
        if (!e) {
            variant = TDG_VARIANT_REG_PREFETCH;
            e = find_entry(*tile, 2, variant, true);
            stages = 2;
        }
    } else if (variant == TDG_VARIANT_REG_PREFETCH && stages == 1) {
        e = find_entry(*tile, 2, variant, true);
        stages = 2;
    } else {
        e = find_entry(*tile, stages, variant, true);
    }
    if (!e) return TDG_ERR_UNSUPPORTED;
    if (e->lds_bytes > kLdsPerCU) return TDG_ERR_UNSUPPORTED;
    if (!offsets_fit(*e, lda, ldb)) return TDG_ERR_UNSUPPORTED;

    if (out) {
        out->entry = e;
        out->variant = variant;
        out->stages = stages;
        out->guarded = guard;
    }
    if (cfg_out) {
        cfg_out->bm = e->bm;
        cfg_out->bn = e->bn;
        cfg_out->bk = cfg_bk(*e);
        cfg_out->waves = cfg_waves(*e);
        cfg_out->lds_stages = stages;
        cfg_out->variant = variant;
    }
    fill_info(*e, variant, stages, M, N, K, guard, info);
    return TDG_OK;
}

// Recent resolutions, so that repeated calls on one shape skip the table
// scans.  The key holds everything resolve() reads: the request, the shape,
// the operands' alignment, whether their last chunks stay in their pages,
// and the leading dimensions (which decide whether the chosen kernel's
// 32-bit per-lane offsets reach every chunk).
struct PlanKey {
    int dtype, variant_req, bm, bn, bk, waves, stages, pipelined_default, vec_ok, end_ok;
    int64_t M, N, K, lda, ldb;
    bool operator==(const PlanKey &o) const { return memcmp(this, &o, sizeof(PlanKey)) == 0; }
};
struct PlanSlot {
    bool used;
    PlanKey key;
    int rc;
    Resolved r;
};
std::mutex g_plan_mutex;
PlanSlot g_plans[16];
unsigned g_plan_next = 0;

int resolve_cached(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                   const void *B, int64_t ldb, const tdg_config &req, bool pipelined_default,
                   Resolved *out) {
    PlanKey key;
    memset(&key, 0, sizeof(key));  // padding too: the key is compared bytewise
    key.dtype = dtype;
    key.variant_req = req.variant;
    key.bm = req.bm;
    key.bn = req.bn;
    key.bk = req.bk;
    key.waves = req.waves;
    key.stages = req.lds_stages;
    key.pipelined_default = pipelined_default ? 1 : 0;
    key.vec_ok = aligned_operands(dtype, A, lda, B, ldb) ? 1 : 0;
    key.end_ok = ends_in_page(dtype, M, N, K, A, lda, B, ldb) ? 1 : 0;
    key.M = M;
    key.N = N;
    key.K = K;
    key.lda = lda;
    key.ldb = ldb;
    {
        std::lock_guard<std::mutex> lock(g_plan_mutex);
        for (const PlanSlot &slot : g_plans)
            if (slot.used && slot.key == key) {
                *out = slot.r;
                return slot.rc;
            }
    }
    const int rc = resolve(dtype, M, N, K, A, lda, B, ldb, key.end_ok != 0, req, pipelined_default, out, nullptr,
                           nullptr);
    std::lock_guard<std::mutex> lock(g_plan_mutex);
    PlanSlot &slot = g_plans[g_plan_next++ % 16];
    slot.used = true;
    slot.key = key;
    slot.rc = rc;
    slot.r = *out;
    return rc;
}

// Launch one GEMM.  With parts > 1 (split K), the kernel writes `parts`
// dense M x N partial products to `ws` and a second kernel sums them into C.
int run(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
        int64_t ldb, void *C, int64_t ldc, void *stream, const tdg_config *cfg,
        bool pipelined_default, int parts = 1, void *ws = nullptr) {
    int rc = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc);
    if (rc != TDG_OK) return rc;
    if (M == 0 || N == 0) return TDG_OK;
    tdg_config req;
    memset(&req, 0, sizeof(req));
    if (cfg) req = *cfg;
    Resolved r;
    memset(&r, 0, sizeof(r));
    rc = resolve_cached(dtype, M, N, K, A, lda, B, ldb, req, pipelined_default, &r);
    if (rc != TDG_OK) return rc;
    rc = device_check();
    if (rc != TDG_OK) return rc;

    const KernelEntry &e = *r.entry;
    tdg::GemmArgs args;
    args.A = (const unsigned char *)A;
    args.B = (const unsigned char *)B;
    args.C = (unsigned char *)C;
    args.lda = lda;
    args.ldb = ldb;
    args.ldc = ldc;
    args.M = (int)M;
    args.N = (int)N;
    args.K = (int)K;
    args.tiles_m = (int)ceil_div(M, e.bm);
    args.tiles_n = (int)ceil_div(N, e.bn);
    args.k_tiles = (int)ceil_div(K, cfg_bk(e));
    args.flags = tdg::debug_flags.load(std::memory_order_relaxed);
    args.k_rotate = k_rotation(dtype, N, K) && !(args.flags & TDG_DEBUG_NO_K_ROTATION) ? 1 : 0;
    // Split K only over whole tiles, and never into an empty part.
    if (parts > args.k_tiles) parts = args.k_tiles > 0 ? args.k_tiles : 1;
    args.k_per_part = parts > 1 ? (int)ceil_div(args.k_tiles, parts) : args.k_tiles;
    if (parts > 1) parts = (int)ceil_div(args.k_tiles, args.k_per_part);
    args.k_parts = parts;
    args.part_stride = 0;
    if (parts > 1) {
        args.C = (unsigned char *)ws;
        args.ldc = N;
        args.part_stride = M * N * 4;
    }
    const int64_t grid = (int64_t)args.tiles_m * args.tiles_n * parts;
    if (grid > INT32_MAX) return TDG_ERR_UNSUPPORTED;

    void *kargs[] = {&args};
    hipError_t err = hipLaunchKernel(e.fn, dim3((unsigned)grid), dim3((unsigned)e.threads), kargs,
                                     0, (hipStream_t)stream);
    if (err != hipSuccess) return TDG_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return TDG_ERR_LAUNCH;
    if (parts > 1) return tdg::launch_sum_parts(dtype, parts, ws, M, N, C, ldc, stream);
    return TDG_OK;
}

// ---------------------------------------------------------------- split K

// Predicted microseconds of the split-K second pass: read parts partial
// products and write C at HBM speed, plus a launch.
double sum_parts_us(int parts, int64_t M, int64_t N) {
    const double bytes = (double)(parts + 1) * (double)M * (double)N * 4.0;
    return 5.0 + bytes / 3.0e6;  // a launch and ~3 TB/s
}

// Split-K plan: the configuration and number of K parts with the least
// predicted time, for products whose tiles leave most compute units idle.
// parts = 1 (no split) unless splitting is predicted at least 10% faster.
// Each part keeps at least two K tiles, so its loop still pipelines.  Part
// counts whose partial products exceed ws_limit bytes are not considered.
int splitk_choose(int dtype, int64_t M, int64_t N, int64_t K, tdg_config *cfg, int *parts,
                  uint64_t ws_limit = UINT64_MAX) {
    tdg_config req;
    memset(&req, 0, sizeof(req));
    memset(cfg, 0, sizeof(*cfg));
    *parts = 1;
    if (M <= 0 || N <= 0 || K <= 0) return TDG_OK;  // nothing to split
    const Choice base = choose_config(dtype, M, N, K, req);
    if (!base.tile) return TDG_ERR_UNSUPPORTED;
    const int es = elem_size(dtype);
    double best_t = -1.0;
    const PerfRow *best_row = nullptr;
    int best_parts = 1;
    for (const PerfRow &r : kPerf) {
        if (r.dtype != dtype || !tile_entry(dtype, r.bm, r.bn, 128, r.waves)) continue;
        const int bk = 128 / es;
        const int64_t k_tiles = ceil_div(K, bk);
        tdg_plan_info fig;
        tile_figures(dtype, r.bm, r.bn, bk, r.waves, r.stages, TDG_VARIANT_DIRECT_LDS, M, N, K, &fig);
        for (int p = 1; p <= 256; p *= 2) {
            if (p > 1 && k_tiles < 2 * p) break;
            const int64_t per = ceil_div(k_tiles, p);
            const int64_t used = ceil_div(k_tiles, per);
            if (used > 1 && tdg::splitk_bytes(used, M, N) > ws_limit) continue;
            double t = predict_us(r, fig.wg_per_cu, fig.grid * used, per * bk);
            if (used > 1) t += sum_parts_us((int)used, M, N);
            if (best_t < 0.0 || t < best_t) {
                best_t = t;
                best_row = &r;
                best_parts = (int)used;
            }
        }
    }
    // the plain plan's own prediction: keep it unless the split is clearly faster
    double plain_t = -1.0;
    for (const PerfRow &r : kPerf) {
        if (r.dtype == dtype && r.bm == base.tile->bm && r.bn == base.tile->bn &&
            r.waves == cfg_waves(*base.tile) && r.stages == base.stages) {
            tdg_plan_info fig;
            tile_figures(dtype, r.bm, r.bn, 128 / es, r.waves, r.stages, TDG_VARIANT_DIRECT_LDS, M, N, K,
                         &fig);
            plain_t = predict_us(r, fig.wg_per_cu, fig.grid, K);
        }
    }
    memset(cfg, 0, sizeof(*cfg));
    if (!best_row || best_parts == 1 || (plain_t > 0.0 && best_t > 0.9 * plain_t)) {
        *parts = 1;
        return TDG_OK;
    }
    cfg->bm = best_row->bm;
    cfg->bn = best_row->bn;
    cfg->bk = 128 / es;
    cfg->waves = best_row->waves;
    cfg->lds_stages = best_row->stages;
    cfg->variant = TDG_VARIANT_AUTO;
    *parts = best_parts;
    return TDG_OK;
}

}  // namespace

namespace tdg {

uint64_t splitk_bytes(int64_t parts, int64_t M, int64_t N) {
    if (parts <= 0 || M <= 0 || N <= 0) return 0;
    const uint64_t one = (uint64_t)M * (uint64_t)N * 4u;
    if (one > UINT64_MAX / (uint64_t)parts) return UINT64_MAX;
    return one * (uint64_t)parts;
}

int validate_gemm(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                  int64_t ldb, const void *C, int64_t ldc) {
    return validate(dtype, M, N, K, A, lda, B, ldb, C, ldc);
}

int run_splitk(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
               int64_t ldb, void *C, int64_t ldc, int parts, void *ws, size_t ws_bytes, void *stream,
               uint64_t auto_limit) {
    int rc = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc);
    if (rc != TDG_OK) return rc;
    if (parts < 0) return TDG_ERR_INVALID_ARG;
    tdg_config cfg;
    memset(&cfg, 0, sizeof(cfg));
    // An empty product (K == 0: C is zero-filled) has nothing to split.
    if (parts == 0 && M > 0 && N > 0 && K > 0) {
        rc = splitk_choose(dtype, M, N, K, &cfg, &parts, auto_limit);
        if (rc != TDG_OK) return rc;
    }
    if (parts <= 1 || M == 0 || N == 0 || K == 0)
        return run(dtype, M, N, K, A, lda, B, ldb, C, ldc, stream, parts <= 1 && cfg.bm ? &cfg : nullptr,
                   true);
    // The workspace: parts dense M x N partial products, 16-byte aligned,
    // apart from A, B and C (a size past 64 bits fits no workspace).
    const uint64_t need = splitk_bytes(parts, M, N);
    if (!ws || need == UINT64_MAX || ws_bytes < need || (uintptr_t)ws % 16) return TDG_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    if (ranges_overlap((uintptr_t)ws, need, (uintptr_t)A, span_bytes(M, K, lda, es)) ||
        ranges_overlap((uintptr_t)ws, need, (uintptr_t)B, span_bytes(K, N, ldb, es)) ||
        ranges_overlap((uintptr_t)ws, need, (uintptr_t)C, span_bytes(M, N, ldc, 4)))
        return TDG_ERR_INVALID_ARG;
    return run(dtype, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg.bm ? &cfg : nullptr, true, parts, ws);
}

}  // namespace tdg

namespace {
using tdg::run_splitk;
}  // namespace

extern "C" {

int gemm_f16f32(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                int64_t ldb, float *C, int64_t ldc, void *stream) {
    tdg_config cfg;
    memset(&cfg, 0, sizeof(cfg));
    cfg.variant = TDG_VARIANT_SINGLE;
    return run(TDG_DTYPE_F16F32, M, N, K, A, lda, B, ldb, C, ldc, stream, &cfg, false);
}

int gemm_i8i32(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda, const int8_t *B,
               int64_t ldb, int32_t *C, int64_t ldc, void *stream) {
    tdg_config cfg;
    memset(&cfg, 0, sizeof(cfg));
    cfg.variant = TDG_VARIANT_SINGLE;
    return run(TDG_DTYPE_I8I32, M, N, K, A, lda, B, ldb, C, ldc, stream, &cfg, false);
}

int gemm_f16f32_pipelined(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                          const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream) {
    return run(TDG_DTYPE_F16F32, M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr, true);
}

int gemm_i8i32_pipelined(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                         const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream) {
    return run(TDG_DTYPE_I8I32, M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr, true);
}

int gemm_f16f32_ex(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                   const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream,
                   const tdg_config *cfg) {
    return run(TDG_DTYPE_F16F32, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, true);
}

int gemm_i8i32_ex(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda, const int8_t *B,
                  int64_t ldb, int32_t *C, int64_t ldc, void *stream, const tdg_config *cfg) {
    return run(TDG_DTYPE_I8I32, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, true);
}

int gemm_f32f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                int64_t ldb, float *C, int64_t ldc, void *stream) {
    tdg_config cfg;
    memset(&cfg, 0, sizeof(cfg));
    cfg.variant = TDG_VARIANT_SINGLE;
    return run(TDG_DTYPE_F32F32, M, N, K, A, lda, B, ldb, C, ldc, stream, &cfg, false);
}

int gemm_f32f32_pipelined(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                          const float *B, int64_t ldb, float *C, int64_t ldc, void *stream) {
    return run(TDG_DTYPE_F32F32, M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr, true);
}

int gemm_f32f32_ex(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                   int64_t ldb, float *C, int64_t ldc, void *stream, const tdg_config *cfg) {
    return run(TDG_DTYPE_F32F32, M, N, K, A, lda, B, ldb, C, ldc, stream, cfg, true);
}

int tdg_plan(int dtype, int64_t M, int64_t N, int64_t K, tdg_config *out, tdg_plan_info *info) {
    if (!dtype_ok(dtype)) return TDG_ERR_INVALID_ARG;
    if (!dims_ok(M, N, K)) return TDG_ERR_INVALID_ARG;
    tdg_config req;
    memset(&req, 0, sizeof(req));
    if (out) req = *out;
    // Planning assumes dense operands (lda = K, ldb = N) at 16-byte aligned
    // addresses whose last chunks stay in their pages; the real call's
    // strides and addresses are judged again when it runs
    // (tdg_plan_operands tells what they make of it).
    const void *aligned = (const void *)(uintptr_t)4096;
    const int64_t lda = K > 0 ? K : 1, ldb = N > 0 ? N : 1;
    return resolve(dtype, M, N, K, aligned, lda, aligned, ldb, true, req, true, nullptr, out, info);
}

int tdg_plan_operands(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                      const void *B, int64_t ldb, tdg_config *out, tdg_plan_info *info) {
    if (!dtype_ok(dtype) || !dims_ok(M, N, K)) return TDG_ERR_INVALID_ARG;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1)) return TDG_ERR_INVALID_ARG;
    if ((M > 0 && K > 0 && !A) || (K > 0 && N > 0 && !B)) return TDG_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    if (!extent_ok(M, lda, es) || !extent_ok(K, ldb, es)) return TDG_ERR_INVALID_ARG;
    tdg_config req;
    memset(&req, 0, sizeof(req));
    if (out) req = *out;
    return resolve(dtype, M, N, K, A, lda, B, ldb, ends_in_page(dtype, M, N, K, A, lda, B, ldb), req, true,
                   nullptr, out, info);
}

int tdg_predict_us(int dtype, int bm, int bn, int waves, int stages, int64_t M, int64_t N, int64_t K,
                   double *us) {
    if (!dtype_ok(dtype) || !dims_ok(M, N, K) || !us) return TDG_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    for (const PerfRow &r : kPerf) {
        if (r.dtype != dtype || r.bm != bm || r.bn != bn || r.waves != waves || r.stages != stages)
            continue;
        tdg_plan_info fig;
        tile_figures(dtype, r.bm, r.bn, 128 / es, r.waves, r.stages, TDG_VARIANT_DIRECT_LDS, M, N, K, &fig);
        *us = predict_us(r, fig.wg_per_cu, fig.grid, K);
        return TDG_OK;
    }
    return TDG_ERR_UNSUPPORTED;
}

int tdg_tile_figures(int dtype, int bm, int bn, int bk, int waves, int stages, int variant,
                     int64_t M, int64_t N, int64_t K, tdg_plan_info *info) {
    if (!dtype_ok(dtype)) return TDG_ERR_INVALID_ARG;
    if (bm <= 0 || bn <= 0 || bk <= 0 || waves <= 0 || waves > 16) return TDG_ERR_INVALID_ARG;
    if (bm > kMaxTileSide || bn > kMaxTileSide || bk > kMaxTileSide) return TDG_ERR_INVALID_ARG;
    if (stages < 1 || stages > 8 || !dims_ok(M, N, K) || !info) return TDG_ERR_INVALID_ARG;
    tile_figures(dtype, bm, bn, bk, waves, stages, variant, M, N, K, info);
    return TDG_OK;
}

int tdg_config_count(int dtype) {
    int count = 0, n = 0;
    const KernelEntry *table = tdg::kernel_table(&count);
    for (int i = 0; i < count; i++)
        if (table[i].dtype == dtype && !table[i].guard) n++;
    return n;
}

int tdg_config_at(int dtype, int index, tdg_config *out) {
    if (!out || index < 0) return TDG_ERR_INVALID_ARG;
    int count = 0, n = 0;
    const KernelEntry *table = tdg::kernel_table(&count);
    for (int i = 0; i < count; i++) {
        const KernelEntry &e = table[i];
        if (e.dtype != dtype || e.guard) continue;
        if (n == index) {
            out->bm = e.bm;
            out->bn = e.bn;
            out->bk = cfg_bk(e);
            out->waves = cfg_waves(e);
            out->lds_stages = e.stages;
            out->variant = e.variant;
            return TDG_OK;
        }
        n++;
    }
    return TDG_ERR_INVALID_ARG;
}

int tdg_splitk_plan(int dtype, int64_t M, int64_t N, int64_t K, int *parts, size_t *workspace_bytes) {
    if (!dtype_ok(dtype) || !parts) return TDG_ERR_INVALID_ARG;
    if (!dims_ok(M, N, K)) return TDG_ERR_INVALID_ARG;
    *parts = 1;
    if (workspace_bytes) *workspace_bytes = 0;
    if (M == 0 || N == 0 || K == 0) return TDG_OK;
    tdg_config cfg;
    const int rc = splitk_choose(dtype, M, N, K, &cfg, parts);
    if (rc != TDG_OK) return rc;
    if (workspace_bytes && *parts > 1) *workspace_bytes = (size_t)tdg::splitk_bytes(*parts, M, N);
    return TDG_OK;
}

int gemm_f16f32_splitk(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                       int64_t ldb, float *C, int64_t ldc, int parts, void *workspace, size_t workspace_bytes,
                       void *stream) {
    return run_splitk(TDG_DTYPE_F16F32, M, N, K, A, lda, B, ldb, C, ldc, parts, workspace, workspace_bytes,
                      stream);
}

int gemm_i8i32_splitk(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda, const int8_t *B,
                      int64_t ldb, int32_t *C, int64_t ldc, int parts, void *workspace, size_t workspace_bytes,
                      void *stream) {
    return run_splitk(TDG_DTYPE_I8I32, M, N, K, A, lda, B, ldb, C, ldc, parts, workspace, workspace_bytes,
                      stream);
}

int gemm_f32f32_splitk(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                       int64_t ldb, float *C, int64_t ldc, int parts, void *workspace, size_t workspace_bytes,
                       void *stream) {
    return run_splitk(TDG_DTYPE_F32F32, M, N, K, A, lda, B, ldb, C, ldc, parts, workspace, workspace_bytes,
                      stream);
}

int tdg_config_resources(int dtype, int index, tdg_kernel_resources *out) {
    if (!out || index < 0 || !dtype_ok(dtype)) return TDG_ERR_INVALID_ARG;
    int count = 0, n = 0;
    const KernelEntry *table = tdg::kernel_table(&count);
    const KernelEntry *e = nullptr;
    for (int i = 0; i < count && !e; i++) {
        if (table[i].dtype != dtype || table[i].guard) continue;
        if (n++ == index) e = &table[i];
    }
    if (!e) return TDG_ERR_INVALID_ARG;
    const int rc = device_check();
    if (rc != TDG_OK) return rc;
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, e->fn) != hipSuccess) return TDG_ERR_LAUNCH;
    int resident = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&resident, e->fn, e->threads, 0) != hipSuccess)
        return TDG_ERR_LAUNCH;
    out->vgprs = attr.numRegs;
    out->spill_bytes = (int)attr.localSizeBytes;
    out->lds_bytes = (int)attr.sharedSizeBytes;
    out->threads = e->threads;
    out->wg_per_cu = resident;
    return TDG_OK;
}

int tdg_set_debug_flags(int flags) {
    if (flags & ~(TDG_DEBUG_POISON_LDS | TDG_DEBUG_NO_K_ROTATION)) return TDG_ERR_INVALID_ARG;
    return tdg::debug_flags.exchange(flags);
}

const char *tdg_status_string(int status) {
    switch (status) {
        case TDG_OK: return "ok";
        case TDG_ERR_INVALID_ARG: return "invalid argument";
        case TDG_ERR_UNSUPPORTED: return "unsupported configuration";
        case TDG_ERR_LAUNCH: return "kernel launch failed";
        case TDG_ERR_NO_DEVICE: return "no gfx950 device";
        case TDG_ERR_SCRATCH: return "partial products exceed the built-in scratch array";
        default: return "unknown status";
    }
}

}  // extern "C"
