/* tdg_c_consumer.c -- a plain C99 program that reaches the GEMM library only
 * through include/tdgemm.h and the HIP runtime's C API: no Python, no C++,
 * no torch.  It is the boundary as a C caller sees it.
 *
 *   tdg_c_consumer host  argument validation, planning, configuration
 *                        tables, status strings and the debug switch; no
 *                        device is needed, because every check runs before
 *                        any HIP call.
 *   tdg_c_consumer gpu   INT8, FP16 and FP32 products on the device, on a
 *                        ragged shape and a whole-tile one, plain, with K
 *                        split through a workspace and through the
 *                        allocation-free entry point, each checked against
 *                        the CPU oracle (liboracle_gemm.so): INT8 bit-exact,
 *                        FP16 and FP32 within 1e-4 * sum |a b|.
 *
 * Prints one line per check and exits non-zero at the first failure. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tdgemm.h"

/* the CPU oracle (tests only) */
int oracle_gemm_i8i64(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                      const int8_t *B, int64_t ldb, int64_t *C, int nthreads);
int oracle_gemm_f16f64(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb, double *C, double *S, int nthreads);
int oracle_gemm_f32f64(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                       const float *B, int64_t ldb, double *C, double *S, int nthreads);

static int failures = 0;

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            printf("FAIL %s:%d: ", __FILE__, __LINE__);   \
            printf(__VA_ARGS__);                          \
            printf("\n");                                 \
            failures++;                                   \
            return 1;                                     \
        }                                                 \
    } while (0)

/* xorshift64*: the test's own input stream */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static int host_checks(void) {
    int8_t dummy[64] = {0};
    const int8_t *a = dummy;
    int32_t *c = (int32_t *)(void *)(dummy + 32);
    tdg_config cfg;
    tdg_plan_info info;

    CHECK(gemm_i8i32(-1, 4, 4, a, 4, a, 4, c, 4, NULL) == TDG_ERR_INVALID_ARG, "negative M");
    CHECK(gemm_i8i32(4, 4, 8, a, 4, a, 4, c, 4, NULL) == TDG_ERR_INVALID_ARG, "lda < K");
    CHECK(gemm_i8i32(4, 4, 4, NULL, 4, a, 4, c, 4, NULL) == TDG_ERR_INVALID_ARG, "NULL A");
    CHECK(gemm_i8i32(4, 4, 4, a, 4, a, 4, (int32_t *)(void *)dummy, 4, NULL) == TDG_ERR_INVALID_ARG,
          "C overlapping A");
    /* an empty A and C may be NULL; B (7 x 5) may not */
    CHECK(gemm_f16f32_pipelined(0, 5, 7, NULL, 7, (const uint16_t *)(const void *)dummy, 5, NULL, 5, NULL) ==
              TDG_OK, "M = 0 is a no-op");
    CHECK(gemm_f16f32_pipelined(0, 5, 7, NULL, 7, NULL, 5, NULL, 5, NULL) == TDG_ERR_INVALID_ARG,
          "NULL B of a non-empty matrix");
    printf("validation ok\n");

    CHECK(tdg_plan(TDG_DTYPE_F16F32, 4096, 4096, 4096, &cfg, &info) == TDG_OK, "plan");
    CHECK(cfg.bm == 256 && cfg.bn == 256 && cfg.variant == TDG_VARIANT_DIRECT_LDS,
          "4096^3 plan %dx%d variant %d", cfg.bm, cfg.bn, cfg.variant);
    CHECK(fabs(info.ratio - 128.0) < 1e-9, "ratio %g", info.ratio);
    CHECK(info.num_tiles == 64 && info.grid == 256, "tiles %lld grid %lld", (long long)info.num_tiles,
          (long long)info.grid);
    printf("plan 4096^3 fp16: %dx%dx%d, %d waves, %d stages, ratio %.0f ok\n", cfg.bm, cfg.bn, cfg.bk,
           cfg.waves, cfg.lds_stages, info.ratio);

    CHECK(tdg_config_count(TDG_DTYPE_I8I32) > 0, "config table");
    CHECK(tdg_config_at(TDG_DTYPE_I8I32, 0, &cfg) == TDG_OK, "config 0");
    CHECK(tdg_config_at(TDG_DTYPE_I8I32, 100000, &cfg) == TDG_ERR_INVALID_ARG, "config index range");
    CHECK(strcmp(tdg_status_string(TDG_OK), "ok") == 0, "status string");
    CHECK(tdg_set_debug_flags(TDG_DEBUG_POISON_LDS) == 0 && tdg_set_debug_flags(0) == TDG_DEBUG_POISON_LDS,
          "debug flags");
    printf("tables, strings and flags ok\n");
    return 0;
}

#define HIP_OK(call) CHECK((call) == hipSuccess, "%s", #call)

/* Random binary16 with exponent 13..16 (|x| in [0.25, 4)), random sign and
 * mantissa; random binary32 in the same range. */
static uint16_t rand_f16(void) {
    uint32_t r = next_u32();
    return (uint16_t)(((r >> 31) << 15) | ((13u + ((r >> 10) & 3u)) << 10) | (r & 0x3FFu));
}
static float rand_f32(void) {
    uint32_t r = next_u32(), bits = ((r >> 31) << 31) | ((125u + ((r >> 23) & 3u)) << 23) | (r & 0x7FFFFFu);
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

static int gpu_case(int dtype, int64_t M, int64_t N, int64_t K) {
    const size_t es = dtype == TDG_DTYPE_I8I32 ? 1 : (dtype == TDG_DTYPE_F16F32 ? 2 : 4);
    const size_t na = (size_t)(M * K), nb = (size_t)(K * N), nc = (size_t)(M * N);
    unsigned char *ha = malloc(na * es), *hb = malloc(nb * es);
    void *hc = malloc(nc * 4);
    double *ref = malloc(nc * sizeof(double)), *sum = malloc(nc * sizeof(double));
    int64_t *iref = malloc(nc * sizeof(int64_t));
    void *da = NULL, *db = NULL, *dc = NULL;
    size_t i;
    int rc;
    CHECK(ha && hb && hc && ref && sum && iref, "host allocation");
    for (i = 0; i < na; i++) {
        if (es == 1) ha[i] = (unsigned char)next_u32();
        else if (es == 2) ((uint16_t *)ha)[i] = rand_f16();
        else ((float *)ha)[i] = rand_f32();
    }
    for (i = 0; i < nb; i++) {
        if (es == 1) hb[i] = (unsigned char)next_u32();
        else if (es == 2) ((uint16_t *)hb)[i] = rand_f16();
        else ((float *)hb)[i] = rand_f32();
    }
    HIP_OK(hipMalloc(&da, na * es));
    HIP_OK(hipMalloc(&db, nb * es));
    HIP_OK(hipMalloc(&dc, nc * 4));
    HIP_OK(hipMemcpy(da, ha, na * es, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(db, hb, nb * es, hipMemcpyHostToDevice));
    if (dtype == TDG_DTYPE_I8I32)
        rc = gemm_i8i32_pipelined(M, N, K, da, K, db, N, dc, N, NULL);
    else if (dtype == TDG_DTYPE_F16F32)
        rc = gemm_f16f32_pipelined(M, N, K, da, K, db, N, dc, N, NULL);
    else
        rc = gemm_f32f32_pipelined(M, N, K, da, K, db, N, dc, N, NULL);
    CHECK(rc == TDG_OK, "gemm dtype %d: %s", dtype, tdg_status_string(rc));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hc, dc, nc * 4, hipMemcpyDeviceToHost));
    if (dtype == TDG_DTYPE_I8I32) {
        CHECK(oracle_gemm_i8i64(M, N, K, (const int8_t *)ha, K, (const int8_t *)hb, N, iref, 0) == 0, "oracle");
        for (i = 0; i < nc; i++)
            CHECK((int64_t)((int32_t *)hc)[i] == iref[i], "int8 element %zu: %d vs %lld", i,
                  ((int32_t *)hc)[i], (long long)iref[i]);
    } else {
        if (dtype == TDG_DTYPE_F16F32)
            rc = oracle_gemm_f16f64(M, N, K, (const uint16_t *)ha, K, (const uint16_t *)hb, N, ref, sum, 0);
        else
            rc = oracle_gemm_f32f64(M, N, K, (const float *)ha, K, (const float *)hb, N, ref, sum, 0);
        CHECK(rc == 0, "oracle");
        for (i = 0; i < nc; i++) {
            const double got = ((float *)hc)[i];
            CHECK(fabs(got - ref[i]) <= 1e-4 * sum[i], "element %zu: %.9g vs %.9g (S %.3g)", i, got, ref[i],
                  sum[i]);
        }
    }
    /* the same product with K split in 3 parts through a hipMalloc workspace:
       INT8 must not change at all, the others stay within the bound */
    if (K >= 3 * 128) {
        void *ws = NULL;
        const size_t wsb = (size_t)3 * (size_t)nc * 4u;
        HIP_OK(hipMalloc(&ws, wsb));
        HIP_OK(hipMemset(dc, 0, nc * 4));
        if (dtype == TDG_DTYPE_I8I32)
            rc = gemm_i8i32_splitk(M, N, K, da, K, db, N, dc, N, 3, ws, wsb, NULL);
        else if (dtype == TDG_DTYPE_F16F32)
            rc = gemm_f16f32_splitk(M, N, K, da, K, db, N, dc, N, 3, ws, wsb, NULL);
        else
            rc = gemm_f32f32_splitk(M, N, K, da, K, db, N, dc, N, 3, ws, wsb, NULL);
        CHECK(rc == TDG_OK, "split-K gemm dtype %d: %s", dtype, tdg_status_string(rc));
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(hc, dc, nc * 4, hipMemcpyDeviceToHost));
        for (i = 0; i < nc; i++) {
            if (dtype == TDG_DTYPE_I8I32) {
                CHECK((int64_t)((int32_t *)hc)[i] == iref[i], "split-K int8 element %zu", i);
            } else {
                const double got = ((float *)hc)[i];
                CHECK(fabs(got - ref[i]) <= 1e-4 * sum[i], "split-K element %zu: %.9g vs %.9g", i, got, ref[i]);
            }
        }
        hipFree(ws);
        /* and through the allocation-free entry point, which needs no
           workspace at all: 3 parts, then the planner's count */
        {
            const int counts[2] = {3, 0};
            int c;
            for (c = 0; c < 2; c++) {
                HIP_OK(hipMemset(dc, 0, nc * 4));
                rc = gemm_splitk_noalloc(dtype, M, N, K, da, K, db, N, dc, N, counts[c], NULL);
                CHECK(rc == TDG_OK, "no-alloc split K dtype %d parts %d: %s", dtype, counts[c],
                      tdg_status_string(rc));
                HIP_OK(hipDeviceSynchronize());
                HIP_OK(hipMemcpy(hc, dc, nc * 4, hipMemcpyDeviceToHost));
                for (i = 0; i < nc; i++) {
                    if (dtype == TDG_DTYPE_I8I32) {
                        CHECK((int64_t)((int32_t *)hc)[i] == iref[i], "no-alloc int8 element %zu", i);
                    } else {
                        const double got = ((float *)hc)[i];
                        CHECK(fabs(got - ref[i]) <= 1e-4 * sum[i], "no-alloc element %zu: %.9g vs %.9g", i, got,
                              ref[i]);
                    }
                }
            }
        }
    }
    printf("gpu dtype %d %lldx%lldx%lld ok\n", dtype, (long long)M, (long long)N, (long long)K);
    hipFree(da);
    hipFree(db);
    hipFree(dc);
    free(ha);
    free(hb);
    free(hc);
    free(ref);
    free(sum);
    free(iref);
    return 0;
}

int main(int argc, char **argv) {
    if (argc != 2 || (strcmp(argv[1], "host") && strcmp(argv[1], "gpu"))) {
        fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
        return 2;
    }
    if (!strcmp(argv[1], "host")) {
        if (host_checks()) return 1;
    } else {
        const int dtypes[3] = {TDG_DTYPE_I8I32, TDG_DTYPE_F16F32, TDG_DTYPE_F32F32};
        int d;
        for (d = 0; d < 3; d++) {
            if (gpu_case(dtypes[d], 300, 290, 333)) return 1;
            if (gpu_case(dtypes[d], 512, 512, 512)) return 1;
        }
    }
    printf("%s checks passed\n", argv[1]);
    return failures ? 1 : 0;
}
