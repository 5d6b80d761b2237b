/*
 * tdgemm.h -- C ABI of the MI355X (gfx950) tiled dense GEMM library.
 *
 * Every entry point computes C = A . B, the plain matrix product ("Pipeline
 * GPU Kernel", Step 2: 2 operations per multiply-add; "Analyze Kernel
 * Bottleneck", Step 1: a GEMM does 2*M*N*K operations), with
 *   A: M x K, row-major, leading dimension lda (elements),
 *   B: K x N, row-major, leading dimension ldb (elements),
 *   C: M x N, row-major, leading dimension ldc (elements), overwritten.
 * FP16 entry points take binary16 inputs as raw 16-bit patterns and write
 * FP32 results accumulated in FP32; INT8 entry points take int8 inputs and
 * write INT32 results accumulated in INT32 (exact while |C| < 2^31, which
 * holds for every K <= 131071); FP32 entry points take binary32 inputs and
 * write FP32 results accumulated in FP32 (the pages' third data type,
 * "Pipeline GPU Kernel", Step 5: FP32 scalar FFMA; on gfx950 it runs on the
 * matrix cores' v_mfma_f32_32x32x2_f32).
 *
 * The K loop runs in tiles of BK elements staged through on-chip LDS:
 *   - the unpipelined entry points run the sequential baseline: load tile t,
 *     barrier, compute on it, barrier ("Pipeline GPU Kernel", Step 1);
 *   - the _pipelined entry points run the prologue / main loop / epilogue
 *     form in which the global load of tile t+1 is in flight while the matrix
 *     cores compute on tile t, with two LDS buffers ("Pipeline GPU Kernel",
 *     Step 3 and Step 4) or a deeper ring of them.  The variant (register
 *     prefetch or direct global-to-LDS) and the ring depth are chosen per
 *     shape by tdg_plan.
 *
 * Pointers A, B, C are DEVICE pointers owned by the caller; the library never
 * allocates, frees or synchronises.  `stream` is a hipStream_t (NULL = the
 * null stream); each call only enqueues work and returns.  Calls are
 * thread-safe.
 *
 * Argument rules (violations return TDG_ERR_INVALID_ARG before any HIP call):
 *   0 <= M, N, K <= 2^31 - 2^16 (the kernels index in 32 bits);
 *   lda >= max(1, K);  ldb >= max(1, N);  ldc >= max(1, N);
 *   a pointer may be NULL only when its matrix is empty;
 *   rows * ld * sizeof(element) of each matrix must fit in int64;
 *   the bytes C spans may not overlap those of A or B.
 * The kernels reach the rows of A and B that one thread loads from with an
 * unsigned 32-bit per-lane byte offset: for the kernel a call runs,
 * (R - 1) * ld * sizeof(T) + (row bytes of one tile) must stay below 2^32,
 * where R is the number of A (or B) tile rows the workgroup's threads cover
 * with their first chunk (at most 128).  Every built kernel accepts
 * lda * sizeof(T) and ldb * sizeof(T) up to 33,818,639 bytes (about 16.9
 * million FP16, 33.8 million INT8 or 8.4 million FP32 elements); a call whose
 * kernel cannot reach its rows returns TDG_ERR_UNSUPPORTED.
 * Degenerate shapes: M == 0 or N == 0 returns TDG_OK and launches nothing;
 * K == 0 writes zeros to C.
 * Any shape and alignment is accepted.  Whole tiles (M, N, K multiples of
 * the tile) run the unchecked kernels: the direct-to-LDS loop at any
 * alignment (its DMA reads 16 bytes from any byte address), the register and
 * sequential loops with 16-byte aligned A and B and lda, ldb multiples of 16
 * bytes.  Ragged shapes run the bounds-checked direct-to-LDS loop: chunks
 * sit on a 16-byte grid from each row's first byte, those that start outside
 * A or B are fetched from a zero block, those that start inside are fetched
 * whole (A's bytes at k >= K are then cleared in LDS), and stores are
 * masked.  When the chunk holding an operand's last byte would reach into
 * another 4 KiB page, the bounds-checked register-prefetch form runs
 * instead: one 16-byte load per chunk at any byte alignment, partial chunks
 * that would leave their page loaded end-anchored and shifted ("Pipeline GPU
 * Kernel", Common Pitfalls: boundary handling with async copies).
 * tdg_plan_operands tells which form a call runs.  Reads stay inside each
 * operand's span -- from its first byte through the 4 KiB page of its last
 * byte, rows and the gaps between them (one allocation, as for any strided
 * view) -- so the operands need no padding.
 * Errors: TDG_ERR_NO_DEVICE when the current device is not gfx950 or no
 * device is present; TDG_ERR_UNSUPPORTED for an explicit configuration that is
 * not built in or does not fit the device; TDG_ERR_LAUNCH when the launch
 * itself fails.
 */
#ifndef TDGEMM_H
#define TDGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TDG_OK = 0,
    TDG_ERR_INVALID_ARG = -1,
    TDG_ERR_UNSUPPORTED = -2,
    TDG_ERR_LAUNCH = -3,
    TDG_ERR_NO_DEVICE = -4,
    TDG_ERR_SCRATCH = -5 /* gemm_splitk_noalloc: partials exceed its scratch */
} tdg_status;

typedef enum {
    TDG_DTYPE_F16F32 = 0, /* binary16 inputs, FP32 accumulate and output */
    TDG_DTYPE_I8I32 = 1,  /* int8 inputs, INT32 accumulate and output */
    TDG_DTYPE_F32F32 = 2  /* binary32 inputs, FP32 accumulate and output */
} tdg_dtype;

typedef enum {
    TDG_VARIANT_AUTO = 0,         /* let tdg_plan choose */
    TDG_VARIANT_SINGLE = 1,       /* sequential load-barrier-compute-barrier */
    TDG_VARIANT_REG_PREFETCH = 2, /* global -> registers for t+1 during compute on t */
    TDG_VARIANT_DIRECT_LDS = 3    /* global -> LDS (LDS-DMA) for t+1 during compute on t */
} tdg_variant;

/* One kernel configuration.  bk is in elements (64 for FP16, 128 for INT8 at
 * the default 128-byte K tile); waves is the wavefront count per workgroup
 * (64 lanes each); lds_stages is the number of LDS tile buffers: 1 for the
 * sequential loop, 1 or 2 for register prefetch, 2 to 8 for direct-to-LDS
 * (a ring with lds_stages - 1 tiles in flight). */
typedef struct {
    int bm, bn, bk, waves, lds_stages, variant;
} tdg_config;

/* What the planner computed for a shape and a configuration.
 *   ratio     -- per-tile compute/load ratio 2*BM*BN*BK / ((BM*BK + BK*BN) *
 *                sizeof(T)) in operations per byte ("Pipeline GPU Kernel",
 *                Step 2);
 *   band      -- 0: ratio < 5, 1: 5 <= ratio <= 20, 2: ratio > 20 (the
 *                pages' decision thresholds, measured on another GPU);
 *   lds_bytes -- LDS per workgroup: lds_stages * (BM*BK + BK*BN) * sizeof(T)
 *                ("Pipeline GPU Kernel", Step 1);
 *   wg_per_cu -- workgroups resident per compute unit, the minimum of the LDS
 *                limit (160 KiB per CU), the wave-slot limit and the register
 *                limit ("Analyze Kernel Bottleneck", Step 3 and Step 6);
 *   num_tiles -- ceil(K / BK), the K-loop trip count;
 *   grid      -- workgroups launched, ceil(M/BM) * ceil(N/BN);
 *   est_regs  -- estimated 32-bit registers per lane for accumulators plus
 *                register staging;
 *   guarded   -- 1 when the shape or alignment needs the bounds-checked form;
 *   need_bytes_per_clk -- bytes per clock per compute unit that must move
 *                from L2 into LDS to keep the matrix cores busy: the CU's
 *                MFMA operations per clock (4096 FP16, 8192 INT8, 256 FP32)
 *                divided by `ratio`;
 *   mfma_per_load -- instruction-count form of the ratio: MFMA instructions
 *                per tile over 16-byte-per-lane wave load instructions per
 *                tile ("Analyze Kernel Bottleneck", Step 4 counts compute and
 *                load instructions per tile);
 *   pipelined -- 1 when the chosen loop overlaps the load of tile t+1 with
 *                compute on tile t; 0 for the sequential form, and for
 *                num_tiles < 2, where the planner chooses the sequential
 *                form ("Pipeline GPU Kernel", Step 1: pipelining needs at
 *                least two K tiles);
 *   k_rotated -- 1 when each tile row walks its K tiles starting at its own
 *                offset (tile row mod num_tiles).  Chosen when all of B fits
 *                in half an XCD's L2 (K * N * sizeof(T) <= 2 MiB): B is then
 *                read from L2 in any order, and the rotation spreads A's
 *                concurrent reads over the HBM channels.  It changes the
 *                FP32 summation order (per tile row), not the product. */
typedef struct {
    double ratio;
    int band;
    size_t lds_bytes;
    int wg_per_cu;
    int64_t num_tiles;
    int64_t grid;
    int est_regs;
    int guarded;
    double need_bytes_per_clk;
    double mfma_per_load;
    int pipelined;
    int k_rotated;
} tdg_plan_info;

/* Sequential (single-buffer) baseline, FP16 -> FP32. */
int gemm_f16f32(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream);
/* Sequential (single-buffer) baseline, INT8 -> INT32. */
int gemm_i8i32(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
               const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream);
/* Software-pipelined K loop over double-buffered (or deeper) LDS tiles,
 * FP16 -> FP32. */
int gemm_f16f32_pipelined(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                          const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream);
/* Software-pipelined K loop over double-buffered (or deeper) LDS tiles,
 * INT8 -> INT32. */
int gemm_i8i32_pipelined(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                         const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream);
/* Sequential baseline and pipelined loop, FP32 -> FP32. */
int gemm_f32f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                int64_t ldb, float *C, int64_t ldc, void *stream);
int gemm_f32f32_pipelined(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                          const float *B, int64_t ldb, float *C, int64_t ldc, void *stream);
/* Explicit configuration (tile, waves, LDS stages, variant), for sweeps and
 * side-by-side comparisons.  cfg == NULL behaves like the _pipelined call.
 * Fields left 0 in cfg are filled by the planner.  A configuration that is
 * not built in returns TDG_ERR_UNSUPPORTED. */
int gemm_f16f32_ex(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                   const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream,
                   const tdg_config *cfg);
int gemm_i8i32_ex(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                  const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream,
                  const tdg_config *cfg);
int gemm_f32f32_ex(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                   const float *B, int64_t ldb, float *C, int64_t ldc, void *stream,
                   const tdg_config *cfg);

/* Split K ("Pipeline GPU Kernel", Step 1: too few tiles leave the loop's
 * overlap, and here the chip, unused).  A product with few C tiles and a long
 * K, say 256 x 256 x 65536, keeps one workgroup per tile and leaves most
 * compute units idle.  These entry points cut K into `parts` slices of whole
 * K tiles: parts workgroups per C tile each compute one slice's partial
 * tile into `workspace`, and a second kernel sums the slices in slice order
 * into C.  The result is deterministic, and exact for INT8.
 *   parts == 0  the planner's choice (tdg_splitk_plan); 1 runs the plain
 *               pipelined GEMM, for which the workspace may be NULL;
 *   workspace   caller-owned device memory of at least parts * M * N * 4
 *               bytes, 16-byte aligned, not overlapping A, B or C;
 *               its contents on return are unspecified.
 * A parts count above the number of K tiles is lowered to it.  Errors as for
 * the other entry points; a missing or short workspace is
 * TDG_ERR_INVALID_ARG.  The two kernels are enqueued on `stream`. */
int gemm_f16f32_splitk(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb, float *C, int64_t ldc, int parts,
                       void *workspace, size_t workspace_bytes, void *stream);
int gemm_i8i32_splitk(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                      const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, int parts,
                      void *workspace, size_t workspace_bytes, void *stream);
int gemm_f32f32_splitk(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                       const float *B, int64_t ldb, float *C, int64_t ldc, int parts,
                       void *workspace, size_t workspace_bytes, void *stream);
/* Split K with no allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same product as gemm_f16f32_splitk,
 * gemm_i8i32_splitk or gemm_f32f32_splitk (dtype = TDG_DTYPE_F16F32,
 * TDG_DTYPE_I8I32 or TDG_DTYPE_F32F32; A, B, C of that entry point's element
 * types), with the partial products kept in a device array of
 * TDG_NOALLOC_SCRATCH_BYTES built into the library instead of a caller's
 * workspace.  The library allocates nothing for it: each GPU holds its own
 * copy of the array from the first call on that GPU until the process ends.
 *   parts == 0  the planner's count among those whose partials fit the
 *               array (1, the plain product, always fits);
 *   parts >= 2  parts * M * N * 4 bytes must not exceed
 *               TDG_NOALLOC_SCRATCH_BYTES, else TDG_ERR_SCRATCH before any
 *               HIP call;
 *   parts == 1  the plain pipelined product.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and may return wrong
 * results; calls on one stream are ordered and safe.  Other errors as for
 * gemm_*_splitk; an unknown dtype is TDG_ERR_INVALID_ARG. */
#define TDG_NOALLOC_SCRATCH_BYTES (32u << 20)
int gemm_splitk_noalloc(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                        const void *B, int64_t ldb, void *C, int64_t ldc, int parts, void *stream);

/* The number of K parts the split-K entry points choose for this product (1
 * when splitting is not predicted to be at least 10% faster) and the
 * workspace they then need (0 for 1 part).  Host-only. */
int tdg_splitk_plan(int dtype, int64_t M, int64_t N, int64_t K, int *parts,
                    size_t *workspace_bytes);

/* Planner.  Chooses the configuration the _pipelined call would run for this
 * dtype and shape (variant = TDG_VARIANT_AUTO), or, when `out` holds a
 * partly filled request on entry (any field non-zero), completes that
 * request.  Among the built direct-to-LDS configurations it takes the one
 * with the least predicted kernel time, from a table of times measured on
 * MI355X against workgroup count and K ("Pipeline GPU Kernel", Step 2: when
 * the compute/load ratio does not settle the choice, build the candidates
 * and measure them); a request outside that table gets the largest tile
 * that still gives every compute unit a workgroup.  Writes the result to
 * *out and its figures to *info (either may be NULL).  Host-only
 * arithmetic: needs no device. */
int tdg_plan(int dtype, int64_t M, int64_t N, int64_t K, tdg_config *out, tdg_plan_info *info);

/* The configuration and form that a _pipelined call (or, with a request in
 * *out, an _ex call) would run on these very operands: tdg_plan judges dense
 * operands at 16-byte aligned addresses, while the caller's addresses and
 * leading dimensions decide the forms.  Whole tiles run unchecked in the
 * direct-to-LDS loop at any alignment (its DMA reads 16 bytes from any byte
 * address); the register and sequential loops run unchecked only with
 * 16-byte aligned rows.  Ragged shapes run the bounds-checked direct-to-LDS
 * loop, except when an operand's last 16-byte chunk (chunks sit on a 16-byte
 * grid from each row's first byte) reaches into a 4 KiB page beyond the
 * operand: that page need not be mapped, and the bounds-checked
 * register-prefetch loop runs instead ("Pipeline GPU Kernel", Common
 * Pitfalls: asynchronous copies need valid sources).  info->guarded gives
 * the form.  A and B are compared, never dereferenced: host-only.
 * TDG_ERR_INVALID_ARG for a bad dtype or size, a leading dimension below
 * the row length, or a NULL operand that is not empty. */
int tdg_plan_operands(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                      const void *B, int64_t ldb, tdg_config *out, tdg_plan_info *info);

/* The planner's predicted kernel time, in microseconds, of one row of its
 * measured-time table -- a built direct-to-LDS configuration with a 128-byte
 * K tile: tile bm x bn, `waves` waves, `stages` LDS buffers -- for an
 * M x N x K product: full rounds of (256 compute units x workgroups per
 * unit) workgroups, then the partial round, each priced from times measured
 * on MI355X against workgroup count and K.  The prediction is positive and
 * non-decreasing in M, N and K.  TDG_ERR_UNSUPPORTED when the table has no
 * such row; TDG_ERR_INVALID_ARG for a bad dtype, size or NULL us.
 * Host-only. */
int tdg_predict_us(int dtype, int bm, int bn, int waves, int stages, int64_t M, int64_t N, int64_t K,
                   double *us);

/* The planner's arithmetic for any tile, built or not: the compute/load
 * ratio and its band, the LDS bytes of `stages` buffers ("Pipeline GPU
 * Kernel", Step 1 and Step 2), the workgroups per MI355X compute unit (LDS,
 * wave-slot and register limits; "Analyze Kernel Bottleneck", Step 3 and
 * Step 6), and num_tiles / grid for an M x N x K product.  bk is in
 * elements; variant only affects the register estimate (register staging).
 * Host-only; returns TDG_ERR_INVALID_ARG for tile sizes outside 1..65536,
 * waves outside 1..16, stages outside 1..8, or M, N, K outside the range
 * every entry point accepts (0 .. 2^31 - 2^16). */
int tdg_tile_figures(int dtype, int bm, int bn, int bk, int waves, int stages, int variant,
                     int64_t M, int64_t N, int64_t K, tdg_plan_info *info);

/* Number of built-in kernel configurations for a dtype, and the i-th one. */
int tdg_config_count(int dtype);
int tdg_config_at(int dtype, int index, tdg_config *out);

/* What the i-th built-in configuration (numbered as by tdg_config_at) costs
 * on the device, as the HIP runtime reports it for its kernel: the measured
 * side of the LDS-budget / occupancy table that tdg_tile_figures predicts
 * ("Analyze Kernel Bottleneck", Step 3 and Step 6: occupancy is limited by
 * LDS, registers and wave slots).
 *   vgprs       -- numRegs of the kernel's attributes (registers per lane);
 *   spill_bytes -- private memory per lane (register spills; 0 when none);
 *   lds_bytes   -- static LDS per workgroup (the ring of lds_stages tiles);
 *   threads     -- workgroup size;
 *   wg_per_cu   -- workgroups resident per compute unit by the runtime's
 *                  occupancy calculation.
 * Needs a gfx950 device (TDG_ERR_NO_DEVICE otherwise); a bad dtype, index or
 * NULL out is TDG_ERR_INVALID_ARG; a failing runtime query TDG_ERR_LAUNCH. */
typedef struct {
    int vgprs, spill_bytes, lds_bytes, threads, wg_per_cu;
} tdg_kernel_resources;
int tdg_config_resources(int dtype, int index, tdg_kernel_resources *out);

/* Human-readable name of a status code (static storage). */
const char *tdg_status_string(int status);

/* ---- Debugging aid: a race screen for the K-loop's buffer discipline
 * ("Pipeline GPU Kernel", Common Pitfalls: a missing wait or barrier, or a
 * wrong buffer index, lets compute read a tile that has not landed).  With
 * TDG_DEBUG_POISON_LDS set, every GEMM launched afterwards first fills its
 * whole LDS ring with 0xFF bytes, so such a read yields NaN (FP16, FP32) or
 * -1 (INT8) and fails a comparison with the oracle, rather than passing on
 * stale LDS contents.  Results of correct kernels are unchanged; the fill
 * costs one pass over LDS per workgroup.  The setting is process-wide and
 * read at launch (a graph captured earlier keeps its own).
 * TDG_DEBUG_NO_K_ROTATION turns the K-tile rotation off (see k_rotated in
 * tdg_plan_info), for comparing the two walks.  Returns the previous flags;
 * unknown bits are rejected with TDG_ERR_INVALID_ARG. */
enum { TDG_DEBUG_POISON_LDS = 1, TDG_DEBUG_NO_K_ROTATION = 2 };
int tdg_set_debug_flags(int flags);

/* ---- Copy / transpose ladder ("fixing GPU kernels by hand", the transpose
 * exercise in four steps).  A rows x cols matrix of 32-bit elements (float;
 * the bits are moved, never computed on) is copied or transposed between
 * device buffers owned by the caller.  Effective bandwidth is the bytes that
 * must move, 2 * rows * cols * 4, over the time.  The copy is the upper bound
 * every transpose is measured against; the methods are the page's ladder on
 * gfx950 (64-lane waves, 64 LDS banks), plus two MI355X steps:
 *   NAIVE         coalesced reads, writes strided by the output row length;
 *   LDS           through a 64 x 64 LDS tile read by columns (every column
 *                 read is a 64-way bank conflict);
 *   LDS_PADDED    the page's fix: one extra word per tile row;
 *   LDS_SWIZZLED  the same without the extra word (column index XOR row);
 *   VEC           16-byte loads and stores on both sides of a swizzled,
 *                 pre-transposed tile (whole tiles of 16-byte aligned
 *                 operands; other tiles take the LDS_SWIZZLED path).
 * AUTO is VEC.  Arguments: rows, cols >= 0 (and below 2^31 - 64);
 * ldi >= max(1, cols); ldo >= max(1, cols) for the copy and >= max(1, rows)
 * for the transpose (out is cols x rows); rows * ld * 4 of each matrix must
 * fit in int64; a pointer may be NULL only when the matrix is empty; out may
 * not overlap in.  Violations return
 * TDG_ERR_INVALID_ARG before any HIP call; an empty matrix returns TDG_OK
 * with no launch; a non-gfx950 device returns TDG_ERR_NO_DEVICE; a failed
 * launch TDG_ERR_LAUNCH.  Asynchronous on `stream`, like the GEMM calls. */
typedef enum {
    TDG_TRANSPOSE_AUTO = 0,
    TDG_TRANSPOSE_NAIVE = 1,
    TDG_TRANSPOSE_LDS = 2,
    TDG_TRANSPOSE_LDS_PADDED = 3,
    TDG_TRANSPOSE_LDS_SWIZZLED = 4,
    TDG_TRANSPOSE_VEC = 5
} tdg_transpose_method;

/* out[i][j] = in[i][j]; out is rows x cols. */
int tdg_copy_f32(int64_t rows, int64_t cols, const float *in, int64_t ldi, float *out,
                 int64_t ldo, void *stream);
/* out[j][i] = in[i][j]; out is cols x rows. */
int tdg_transpose_f32(int method, int64_t rows, int64_t cols, const float *in, int64_t ldi,
                      float *out, int64_t ldo, void *stream);

/* ---- Measured compute ceiling ("Analyze Kernel Bottleneck", Step 2: set
 * achieved throughput against what the hardware sustains).  Launches a kernel
 * that issues only the GEMM's MFMA instruction (v_mfma_f32_32x32x16_f16,
 * v_mfma_i32_32x32x32_i8 or v_mfma_f32_32x32x2_f32) with changing
 * pseudo-random operands and no memory
 * traffic: 512 workgroups of 4 waves (two waves per SIMD on 256 CUs), each
 * wave `iters` x 8 MFMAs on eight independent accumulators (80000 iters of
 * the FP16 MFMA is about 20 ms on MI355X).  iters must be a
 * non-negative multiple of 4.  `sink` is a device buffer of
 * tdg_mfma_probe_sink_floats() floats the kernel writes (so the work is not
 * optimised away).  Returns TDG_ERR_INVALID_ARG for a bad dtype, iters or a
 * NULL sink; TDG_ERR_NO_DEVICE off gfx950.  tdg_mfma_probe_ops gives the
 * operations one launch performs (2 * 32 * 32 * k per MFMA, k = 16, 32 or 2),
 * or -1 for bad arguments; time a launch and divide. */
int tdg_mfma_probe(int dtype, int64_t iters, float *sink, void *stream);
int64_t tdg_mfma_probe_ops(int dtype, int64_t iters);
int64_t tdg_mfma_probe_sink_floats(void);

/* The measured LDS read rate ("Analyze Kernel Bottleneck", Step 2: compare
 * with what the hardware delivers): one 8-wave workgroup per compute unit
 * reads its 64 KiB of LDS `iters` x 8 times per thread, without bank
 * conflicts, with mode 0 = 16-byte reads (ds_read_b128, the GEMM's A
 * fragments), 1 = transposing 8-byte reads (ds_read_b64_tr_b16, its B
 * fragments), 2 = plain 8-byte reads (ds_read_b64).  `out` is a device
 * array of 512 uint32: out[w] receives workgroup w's shader cycles
 * (s_memtime), out[256 + w] a value of its reads.  tdg_lds_probe_bytes
 * gives the bytes one workgroup reads (-1 for a bad mode or iters), so
 * bytes / cycles is the per-CU rate per clock.  TDG_ERR_INVALID_ARG for a
 * bad mode, negative iters or NULL out; TDG_ERR_NO_DEVICE off gfx950. */
int tdg_lds_probe(int mode, int64_t iters, uint32_t *out, void *stream);
int64_t tdg_lds_probe_bytes(int mode, int64_t iters);

#ifdef __cplusplus
}
#endif

#endif /* TDGEMM_H */
