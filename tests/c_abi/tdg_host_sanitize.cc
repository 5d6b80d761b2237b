// tdg_host_sanitize.cc -- drives every host-side path of the C ABI (argument
// validation, the planner and its plan cache, split-K planning, the tile
// arithmetic, status strings, debug flags) over a broad set of arguments,
// valid and not, from several threads at once.  It is built against a copy
// of the library compiled host-only with AddressSanitizer and
// UndefinedBehaviorSanitizer, so an out-of-bounds table read, a signed
// overflow in the size arithmetic or a data-structure bug in the plan cache
// stops the run with a report.
//
// No kernel is ever launched: calls that pass validation are made only when
// the HIP runtime reports no device, where they stop at the device check
// (TDG_ERR_NO_DEVICE) after planning.  Operand addresses are made-up
// integers: the host code compares them, never dereferences them.
//
// Prints "sanitized host checks passed" and exits 0, or exits non-zero.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "tdgemm.h"

namespace {

std::atomic<int> g_fail{0};

#define EXPECT(cond, ...)                                          \
    do {                                                           \
        if (!(cond)) {                                             \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__);       \
            std::printf(__VA_ARGS__);                              \
            std::printf("\n");                                     \
            g_fail++;                                              \
        }                                                          \
    } while (0)

const int64_t kMaxDim = (int64_t(1) << 31) - (int64_t(1) << 16);

const int64_t kDims[] = {0, 1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129,
                         255, 256, 257, 1000, 1023, 1024, 1025, 4095, 4096, 4097, 8192,
                         65536, 1 << 20, kMaxDim - 1, kMaxDim};
const int kNumDims = sizeof(kDims) / sizeof(kDims[0]);

uint64_t g_rng = 0x243F6A8885A308D3ull;
uint64_t next_u64() {
    g_rng ^= g_rng >> 12;
    g_rng ^= g_rng << 25;
    g_rng ^= g_rng >> 27;
    return g_rng * 0x2545F4914F6CDD1Dull;
}
int64_t pick_dim() { return kDims[next_u64() % kNumDims]; }
int64_t small_dim() { return (int64_t)(next_u64() % 5000); }

int elem_size(int dtype) { return dtype == TDG_DTYPE_I8I32 ? 1 : (dtype == TDG_DTYPE_F16F32 ? 2 : 4); }

bool status_known(int rc) {
    return rc == TDG_OK || rc == TDG_ERR_INVALID_ARG || rc == TDG_ERR_UNSUPPORTED || rc == TDG_ERR_LAUNCH ||
           rc == TDG_ERR_NO_DEVICE || rc == TDG_ERR_SCRATCH;
}

void check_plan_result(int rc, const tdg_config &c, const tdg_plan_info &info, int64_t M, int64_t N, int64_t K) {
    EXPECT(status_known(rc), "unknown status %d", rc);
    if (rc != TDG_OK) return;
    EXPECT(c.bm > 0 && c.bn > 0 && c.bk > 0 && c.waves > 0, "plan %" PRId64 "x%" PRId64 "x%" PRId64 " empty cfg", M, N, K);
    EXPECT(c.lds_stages >= 1 && c.lds_stages <= 8, "stages %d", c.lds_stages);
    EXPECT(c.variant >= TDG_VARIANT_SINGLE && c.variant <= TDG_VARIANT_DIRECT_LDS, "variant %d", c.variant);
    EXPECT(info.lds_bytes > 0 && info.lds_bytes <= 160u * 1024u, "lds %zu", info.lds_bytes);
    EXPECT(info.wg_per_cu >= 1, "wg_per_cu %d", info.wg_per_cu);
    EXPECT(info.ratio > 0 && std::isfinite(info.ratio), "ratio %g", info.ratio);
    EXPECT(info.num_tiles == (K + c.bk - 1) / c.bk, "num_tiles %" PRId64, info.num_tiles);
    EXPECT(info.grid == ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn), "grid %" PRId64, info.grid);
}

// The planner for every dtype over the dimension set, plain and with each
// built configuration's fields as a partial request, plus malformed ones.
void planner_sweep() {
    for (int dtype = -1; dtype <= 3; dtype++) {
        const int count = tdg_config_count(dtype);
        if (dtype < 0 || dtype > 2) {
            EXPECT(count <= 0, "config count for dtype %d", dtype);
            tdg_config c;
            EXPECT(tdg_plan(dtype, 4, 4, 4, &c, nullptr) == TDG_ERR_INVALID_ARG, "bad dtype plan");
            continue;
        }
        EXPECT(count > 0, "no configs for dtype %d", dtype);
        tdg_config none;
        EXPECT(tdg_config_at(dtype, -1, &none) == TDG_ERR_INVALID_ARG, "index -1");
        EXPECT(tdg_config_at(dtype, count, &none) == TDG_ERR_INVALID_ARG, "index count");
        EXPECT(tdg_config_at(dtype, 0, nullptr) == TDG_ERR_INVALID_ARG, "NULL out");
        for (int a = 0; a < kNumDims; a++)
            for (int b = 0; b < kNumDims; b += 3)
                for (int k = 0; k < kNumDims; k += 4) {
                    const int64_t M = kDims[a], N = kDims[b], K = kDims[k];
                    tdg_config c;
                    tdg_plan_info info;
                    std::memset(&c, 0, sizeof(c));
                    std::memset(&info, 0, sizeof(info));
                    const int rc = tdg_plan(dtype, M, N, K, &c, &info);
                    check_plan_result(rc, c, info, M, N, K);
                    // NULL outputs are allowed
                    tdg_plan(dtype, M, N, K, nullptr, nullptr);
                    tdg_plan(dtype, M, N, K, nullptr, &info);
                }
        for (int i = 0; i < count; i++) {
            tdg_config full;
            EXPECT(tdg_config_at(dtype, i, &full) == TDG_OK, "config %d", i);
            for (int mask = 1; mask < 64; mask++) {
                tdg_config req;
                std::memset(&req, 0, sizeof(req));
                if (mask & 1) req.bm = full.bm;
                if (mask & 2) req.bn = full.bn;
                if (mask & 4) req.bk = full.bk;
                if (mask & 8) req.waves = full.waves;
                if (mask & 16) req.lds_stages = full.lds_stages;
                if (mask & 32) req.variant = full.variant;
                const int64_t M = small_dim(), N = small_dim(), K = small_dim();
                tdg_plan_info info;
                std::memset(&info, 0, sizeof(info));
                tdg_config c = req;
                const int rc = tdg_plan(dtype, M, N, K, &c, &info);
                check_plan_result(rc, c, info, M, N, K);
                if (rc == TDG_OK && mask == 63 && M > 0 && N > 0 && K > 0)
                    EXPECT(c.bm == full.bm && c.bn == full.bn && c.bk == full.bk && c.waves == full.waves,
                           "full request %d changed", i);
            }
        }
        const tdg_config bad[] = {{7, 0, 0, 0, 0, 0},  {0, 0, 0, 3, 0, 0},  {0, 0, 0, 0, 9, 0},
                                  {0, 0, 0, 0, 0, 5},  {0, 0, 0, 0, 0, -1}, {0, 0, 0, 0, -2, 0},
                                  {-64, 0, 0, 0, 0, 0}, {0, 0, 33, 0, 0, 0}, {512, 512, 0, 0, 0, 0},
                                  {0, 0, 0, 0, 1, TDG_VARIANT_DIRECT_LDS},
                                  {0, 0, 0, 0, 3, TDG_VARIANT_REG_PREFETCH},
                                  {0, 0, 0, 0, 2, TDG_VARIANT_SINGLE}};
        for (const tdg_config &b : bad) {
            tdg_config c = b;
            tdg_plan_info info;
            const int rc = tdg_plan(dtype, 300, 300, 300, &c, &info);
            EXPECT(rc == TDG_ERR_INVALID_ARG || rc == TDG_ERR_UNSUPPORTED || rc == TDG_OK,
                   "bad request status %d", rc);
        }
    }
}

// tdg_plan_operands at every byte offset of a chunk and near page ends.
void operands_sweep() {
    const uintptr_t base = (uintptr_t)1 << 40;
    for (int dtype = 0; dtype <= 2; dtype++) {
        const int es = elem_size(dtype);
        for (int iter = 0; iter < 4000; iter++) {
            const int64_t M = (iter % 7 == 0) ? pick_dim() % 70000 : small_dim();
            const int64_t N = (iter % 5 == 0) ? pick_dim() % 70000 : small_dim();
            const int64_t K = small_dim();
            const int64_t lda = (K > 1 ? K : 1) + (int64_t)(next_u64() % 40);
            const int64_t ldb = (N > 1 ? N : 1) + (int64_t)(next_u64() % 40);
            const uintptr_t pa = base + (next_u64() % 8192) * 16 + (next_u64() % 16) / es * es;
            const uintptr_t pb = base + ((uintptr_t)1 << 36) + 4096 - (next_u64() % 64) * es;
            tdg_config c;
            tdg_plan_info info;
            std::memset(&c, 0, sizeof(c));
            const int rc = tdg_plan_operands(dtype, M, N, K, (const void *)pa, lda, (const void *)pb, ldb, &c, &info);
            check_plan_result(rc, c, info, M, N, K);
            EXPECT(rc == TDG_OK || rc == TDG_ERR_UNSUPPORTED, "operands status %d", rc);
        }
        tdg_config c;
        EXPECT(tdg_plan_operands(dtype, 4, 4, 4, nullptr, 4, (const void *)base, 4, &c, nullptr) ==
                   TDG_ERR_INVALID_ARG, "NULL A");
        EXPECT(tdg_plan_operands(dtype, 4, 4, 8, (const void *)base, 4, (const void *)base, 4, &c, nullptr) ==
                   TDG_ERR_INVALID_ARG, "lda < K");
        EXPECT(tdg_plan_operands(dtype, -1, 4, 4, (const void *)base, 4, (const void *)base, 4, &c, nullptr) ==
                   TDG_ERR_INVALID_ARG, "negative M");
        EXPECT(tdg_plan_operands(dtype, kMaxDim, 4, kMaxDim, (const void *)base, INT64_MAX / 2,
                                 (const void *)base, 4, &c, nullptr) == TDG_ERR_INVALID_ARG,
               "extent overflow");
    }
}

// The tile arithmetic and the time model over tiles, built or not.
void figures_sweep() {
    for (int dtype = -1; dtype <= 3; dtype++)
        for (int bm = -32; bm <= 512; bm += 32)
            for (int bn = 0; bn <= 512; bn += 64)
                for (int waves = 0; waves <= 16; waves += 4)
                    for (int stages = 0; stages <= 9; stages += 3) {
                        tdg_plan_info info;
                        const int rc = tdg_tile_figures(dtype, bm, bn, 64, waves, stages, 1 + (bm & 3) % 3,
                                                        pick_dim(), pick_dim(), pick_dim(), &info);
                        EXPECT(status_known(rc), "figures status %d", rc);
                        double us = -1;
                        const int rp = tdg_predict_us(dtype, bm, bn, waves, stages, small_dim(), small_dim(),
                                                      small_dim(), &us);
                        EXPECT(status_known(rp), "predict status %d", rp);
                        if (rp == TDG_OK) EXPECT(us > 0 && std::isfinite(us), "predict %g", us);
                    }
    // Where the table has a row, the prediction never falls as M, N or K grow.
    for (int dtype = 0; dtype <= 2; dtype++) {
        for (int i = 0; i < tdg_config_count(dtype); i++) {
            tdg_config c;
            tdg_config_at(dtype, i, &c);
            double prev = 0;
            for (int64_t d = 1; d <= (int64_t)1 << 16; d = d * 3 / 2 + 1) {
                double us;
                if (tdg_predict_us(dtype, c.bm, c.bn, c.waves, c.lds_stages, d, d, d, &us) != TDG_OK) break;
                EXPECT(us >= prev, "prediction fell at %" PRId64, d);
                prev = us;
            }
        }
        int parts = -1;
        size_t ws = 1;
        for (int it = 0; it < 3000; it++) {
            const int64_t M = pick_dim() % 9000, N = pick_dim() % 9000, K = pick_dim();
            const int rc = tdg_splitk_plan(dtype, M, N, K, &parts, &ws);
            EXPECT(status_known(rc), "splitk status %d", rc);
            if (rc == TDG_OK) {
                EXPECT(parts >= 1, "parts %d", parts);
                EXPECT((parts == 1 && ws == 0) || ws == (size_t)parts * (size_t)M * (size_t)N * 4u,
                       "workspace %zu for %d parts", ws, parts);
            }
        }
        EXPECT(tdg_splitk_plan(dtype, 4, 4, 4, nullptr, &ws) == TDG_ERR_INVALID_ARG, "NULL parts");
    }
    EXPECT(tdg_mfma_probe_ops(7, 4) < 0 && tdg_mfma_probe_ops(0, 3) < 0, "probe ops");
    EXPECT(tdg_lds_probe_bytes(3, 1) < 0 && tdg_lds_probe_bytes(0, -1) < 0, "lds probe bytes");
    for (int s = -10; s <= 2; s++) EXPECT(tdg_status_string(s) != nullptr, "status string %d", s);
    EXPECT(tdg_set_debug_flags(8) == TDG_ERR_INVALID_ARG, "unknown debug bit");
}

// Random and extreme arguments for every host-only entry point: whatever
// they are, the calls return a status, and the sanitizers see no undefined
// arithmetic on the way.
void extreme_fuzz() {
    const int64_t v64[] = {0, 1, -1, 2, 63, 64, 65, 255, 256, 257, 4095, 4096, 4097, 65535, 65536, 65537,
                           (int64_t)1 << 20, kMaxDim - 1, kMaxDim, kMaxDim + 1, (int64_t)1 << 32, (int64_t)1 << 40,
                           INT64_MAX, INT64_MIN, INT32_MAX, INT32_MIN};
    const int nv = sizeof(v64) / sizeof(v64[0]);
    auto any64 = [&]() { return (next_u64() & 1) ? v64[next_u64() % nv] : (int64_t)(next_u64() % 100000); };
    auto any32 = [&]() {
        const int64_t v = any64();
        return (int)(v > INT32_MAX ? INT32_MAX : v < INT32_MIN ? INT32_MIN : v);
    };
    for (int it = 0; it < 60000; it++) {
        const int dtype = (int)(next_u64() % 5) - 1;
        tdg_plan_info info;
        tdg_config c;
        std::memset(&c, 0, sizeof(c));
        if (next_u64() & 1) {
            c.bm = any32(); c.bn = any32(); c.bk = any32(); c.waves = any32();
            c.lds_stages = any32(); c.variant = any32();
        }
        int rc = tdg_plan(dtype, any64(), any64(), any64(), &c, &info);
        EXPECT(status_known(rc), "plan status %d", rc);
        std::memset(&c, 0, sizeof(c));
        rc = tdg_plan_operands(dtype, any64(), any64(), any64(), (const void *)(uintptr_t)next_u64(), any64(),
                               (const void *)(uintptr_t)next_u64(), any64(), &c, &info);
        EXPECT(status_known(rc), "plan_operands status %d", rc);
        rc = tdg_tile_figures(dtype, any32(), any32(), any32(), any32(), any32(), any32(), any64(), any64(), any64(),
                              &info);
        EXPECT(status_known(rc), "figures status %d", rc);
        double us;
        rc = tdg_predict_us(dtype, any32(), any32(), any32(), any32(), any64(), any64(), any64(), &us);
        EXPECT(status_known(rc), "predict status %d", rc);
        int parts;
        size_t ws;
        rc = tdg_splitk_plan(dtype, any64(), any64(), any64(), &parts, &ws);
        EXPECT(status_known(rc), "splitk_plan status %d", rc);
        (void)tdg_mfma_probe_ops(dtype, any64());
        (void)tdg_lds_probe_bytes(dtype, any64());
    }
}

// Arguments every entry point must reject before any HIP call.
void invalid_calls() {
    const uintptr_t a = (uintptr_t)1 << 40, b = a + ((uintptr_t)1 << 36), c = a + ((uintptr_t)1 << 38);
    const void *A = (const void *)a, *B = (const void *)b;
    void *C = (void *)c;
    struct Case { int64_t M, N, K, lda, ldb, ldc; const void *A, *B; void *C; };
    const Case cases[] = {
        {-1, 4, 4, 4, 4, 4, A, B, C},       {4, -1, 4, 4, 4, 4, A, B, C},
        {4, 4, -1, 4, 4, 4, A, B, C},       {kMaxDim + 1, 4, 4, 4, 4, 4, A, B, C},
        {4, 4, 8, 4, 4, 4, A, B, C},        {4, 8, 4, 4, 4, 8, A, B, C},
        {4, 8, 4, 4, 8, 4, A, B, C},        {4, 4, 4, 4, 4, 4, nullptr, B, C},
        {4, 4, 4, 4, 4, 4, A, nullptr, C},  {4, 4, 4, 4, 4, 4, A, B, nullptr},
        {4, 4, 4, 4, 4, 4, A, B, (void *)a}, {kMaxDim, kMaxDim, 4, 4, kMaxDim, INT64_MAX / 4, A, B, C},
    };
    for (const Case &k : cases) {
        int rcs[] = {
            gemm_f16f32(k.M, k.N, k.K, (const uint16_t *)k.A, k.lda, (const uint16_t *)k.B, k.ldb, (float *)k.C, k.ldc, nullptr),
            gemm_i8i32(k.M, k.N, k.K, (const int8_t *)k.A, k.lda, (const int8_t *)k.B, k.ldb, (int32_t *)k.C, k.ldc, nullptr),
            gemm_f32f32(k.M, k.N, k.K, (const float *)k.A, k.lda, (const float *)k.B, k.ldb, (float *)k.C, k.ldc, nullptr),
            gemm_f16f32_pipelined(k.M, k.N, k.K, (const uint16_t *)k.A, k.lda, (const uint16_t *)k.B, k.ldb, (float *)k.C, k.ldc, nullptr),
            gemm_i8i32_pipelined(k.M, k.N, k.K, (const int8_t *)k.A, k.lda, (const int8_t *)k.B, k.ldb, (int32_t *)k.C, k.ldc, nullptr),
            gemm_f32f32_pipelined(k.M, k.N, k.K, (const float *)k.A, k.lda, (const float *)k.B, k.ldb, (float *)k.C, k.ldc, nullptr),
            gemm_f16f32_ex(k.M, k.N, k.K, (const uint16_t *)k.A, k.lda, (const uint16_t *)k.B, k.ldb, (float *)k.C, k.ldc, nullptr, nullptr),
            gemm_i8i32_ex(k.M, k.N, k.K, (const int8_t *)k.A, k.lda, (const int8_t *)k.B, k.ldb, (int32_t *)k.C, k.ldc, nullptr, nullptr),
            gemm_f32f32_ex(k.M, k.N, k.K, (const float *)k.A, k.lda, (const float *)k.B, k.ldb, (float *)k.C, k.ldc, nullptr, nullptr),
            gemm_f16f32_splitk(k.M, k.N, k.K, (const uint16_t *)k.A, k.lda, (const uint16_t *)k.B, k.ldb, (float *)k.C, k.ldc, 0, nullptr, 0, nullptr),
            gemm_i8i32_splitk(k.M, k.N, k.K, (const int8_t *)k.A, k.lda, (const int8_t *)k.B, k.ldb, (int32_t *)k.C, k.ldc, 0, nullptr, 0, nullptr),
            gemm_f32f32_splitk(k.M, k.N, k.K, (const float *)k.A, k.lda, (const float *)k.B, k.ldb, (float *)k.C, k.ldc, 0, nullptr, 0, nullptr),
            gemm_splitk_noalloc(TDG_DTYPE_F16F32, k.M, k.N, k.K, k.A, k.lda, k.B, k.ldb, k.C, k.ldc, 0, nullptr),
        };
        for (int rc : rcs) EXPECT(rc == TDG_ERR_INVALID_ARG, "invalid call returned %d", rc);
    }
    EXPECT(gemm_splitk_noalloc(9, 4, 4, 4, A, 4, B, 4, C, 4, 0, nullptr) == TDG_ERR_INVALID_ARG, "noalloc dtype");
    // parts * M * N * 4 past 64 bits must not wrap into a size that fits
    for (int parts : {1 << 28, (1 << 28) + 1, 0x7FFFFFFF}) {
        const int64_t M = 1 << 17, N = 1 << 17, K = 1024;
        void *W = (void *)((uintptr_t)1 << 45);
        EXPECT(gemm_f16f32_splitk(M, N, K, (const uint16_t *)A, K, (const uint16_t *)B, N, (float *)C, N, parts, W,
                                  16, nullptr) == TDG_ERR_INVALID_ARG, "wrapped workspace size, %d parts", parts);
        EXPECT(gemm_splitk_noalloc(TDG_DTYPE_F16F32, M, N, K, A, K, B, N, C, N, parts, nullptr) == TDG_ERR_SCRATCH,
               "wrapped scratch size, %d parts", parts);
    }
    EXPECT(gemm_f16f32_splitk(4, 4, 4, (const uint16_t *)A, 4, (const uint16_t *)B, 4, (float *)C, 4, -1,
                              nullptr, 0, nullptr) == TDG_ERR_INVALID_ARG, "negative parts");
    EXPECT(tdg_copy_f32(-1, 4, (const float *)A, 4, (float *)C, 4, nullptr) == TDG_ERR_INVALID_ARG, "copy rows");
    EXPECT(tdg_transpose_f32(99, 4, 4, (const float *)A, 4, (float *)C, 4, nullptr) == TDG_ERR_INVALID_ARG,
           "transpose method");
    EXPECT(tdg_transpose_f32(TDG_TRANSPOSE_AUTO, 4, 4, (const float *)A, 4, (float *)A, 4, nullptr) ==
               TDG_ERR_INVALID_ARG, "transpose overlap");
}

// Valid arguments with made-up addresses: each call plans (through the plan
// cache) and then stops at the device check.  Only where no device exists.
void valid_calls_without_device(int thread) {
    uint64_t s = 0x9E3779B97F4A7C15ull * (uint64_t)(thread + 1);
    for (int it = 0; it < 1500; it++) {
        s ^= s >> 12; s ^= s << 25; s ^= s >> 27;
        const uint64_t r = s * 0x2545F4914F6CDD1Dull;
        const int64_t M = 1 + (int64_t)(r % 3000), N = 1 + (int64_t)((r >> 16) % 3000), K = 1 + (int64_t)((r >> 32) % 3000);
        const uintptr_t a = ((uintptr_t)1 << 40) + (r & 15), b = ((uintptr_t)1 << 41) + ((r >> 4) & 15);
        const uintptr_t c = ((uintptr_t)1 << 42);
        const int64_t lda = K + (int64_t)((r >> 8) % 3), ldb = N + (int64_t)((r >> 12) % 3);
        int rc;
        switch (it % 6) {
        case 0: rc = gemm_f16f32_pipelined(M, N, K, (const uint16_t *)a, lda, (const uint16_t *)b, ldb, (float *)c, N, nullptr); break;
        case 1: rc = gemm_i8i32_pipelined(M, N, K, (const int8_t *)a, lda, (const int8_t *)b, ldb, (int32_t *)c, N, nullptr); break;
        case 2: rc = gemm_f32f32(M, N, K, (const float *)a, lda, (const float *)b, ldb, (float *)c, N, nullptr); break;
        case 3: {
            tdg_config cfg;
            tdg_config_at(TDG_DTYPE_I8I32, (int)(r % (uint64_t)tdg_config_count(TDG_DTYPE_I8I32)), &cfg);
            rc = gemm_i8i32_ex(M, N, K, (const int8_t *)a, lda, (const int8_t *)b, ldb, (int32_t *)c, N, nullptr, &cfg);
            break;
        }
        case 4: rc = gemm_f16f32_splitk(M, N, K, (const uint16_t *)a, lda, (const uint16_t *)b, ldb, (float *)c, N, 0,
                                        (void *)((uintptr_t)1 << 43), (size_t)1 << 40, nullptr); break;
        default: rc = gemm_splitk_noalloc(TDG_DTYPE_F32F32, M, N, K, (const void *)a, lda, (const void *)b, ldb,
                                          (void *)c, N, 0, nullptr); break;
        }
        EXPECT(rc == TDG_ERR_NO_DEVICE || rc == TDG_ERR_UNSUPPORTED || rc == TDG_ERR_SCRATCH,
               "thread %d call %d returned %d", thread, it, rc);
    }
}

}  // namespace

int main() {
    if (const char *seed = std::getenv("TDG_FUZZ_SEED")) g_rng ^= std::strtoull(seed, nullptr, 10) * 0x9E3779B97F4A7C15ull;
    int devices = 0;
    const bool no_device = hipGetDeviceCount(&devices) != hipSuccess || devices == 0;
    planner_sweep();
    operands_sweep();
    figures_sweep();
    extreme_fuzz();
    invalid_calls();
    std::vector<std::thread> pool;
    for (int t = 0; t < 8; t++)
        pool.emplace_back([t, no_device] {
            for (int it = 0; it < 200; it++) {
                tdg_config c;
                tdg_plan_info info;
                std::memset(&c, 0, sizeof(c));
                tdg_plan(it % 3, 100 + 37 * it, 64 + 11 * t, 4096, &c, &info);
                tdg_plan_operands(it % 3, 100 + 37 * it, 64 + 11 * t, 999, (const void *)(uintptr_t)(4096 + t),
                                  1000, (const void *)(uintptr_t)(1 << 30), 64 + 11 * t, &c, &info);
            }
            if (no_device) valid_calls_without_device(t);
        });
    for (std::thread &th : pool) th.join();
    if (g_fail.load()) {
        std::printf("%d failures\n", g_fail.load());
        return 1;
    }
    std::printf("sanitized host checks passed (%s)\n", no_device ? "with planned calls" : "device present: planned calls skipped");
    return 0;
}
