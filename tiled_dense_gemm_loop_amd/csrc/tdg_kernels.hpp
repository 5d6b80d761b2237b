// tdg_kernels.hpp -- gfx950 (CDNA4) tiled dense GEMM kernels, C = A . B.
//
// One kernel template covers the sequential baseline and the two pipelined
// variants of "Pipeline GPU Kernel":
//   VAR_SINGLE  -- Step 1's sequential K loop: load tile t to registers, wait,
//                  barrier, write LDS, barrier, compute on it.
//   VAR_REG     -- Step 2/3's register-prefetch variant: the global loads of
//                  tile t+1 go to registers and are in flight while the matrix
//                  cores work on tile t; the registers are then drained into
//                  the other LDS buffer (STAGES = 2), or, with STAGES = 1,
//                  into the same buffer after a barrier (Step 1, "Expected
//                  result on failure": register-only prefetch).
//   VAR_DIRECT  -- Step 2/3's asynchronous-copy variant, done with gfx950's
//                  global-to-LDS DMA (global_load_lds_dwordx4): tiles go
//                  straight into LDS without passing through registers;
//                  "wait for the copies" is s_waitcnt vmcnt followed by the
//                  barrier.  With STAGES = 2 this is the pages' double
//                  buffer; STAGES > 2 turns it into a ring with STAGES - 1
//                  tiles in flight and partial vmcnt waits.
// All three share the prologue / main loop / epilogue shape of Step 3 and the
// buffer discipline of Step 3's failure note: compute reads buffer t % S,
// loads write buffer (t + 1) % S, the epilogue computes buffer
// (num_tiles - 1) % S.
//
// GUARD builds the bounds-checked form of each loop (ragged shapes): the
// sequential and register loops check only the edge tiles, with one 16-byte
// load per chunk at any alignment and a correction of partial chunks after
// they land; the direct-to-LDS loop fetches out-of-range 16-byte chunks from
// a zero block.
//
// Tile micro-kernel: each wave owns a (BM/WM) x (BN/WN) block of C held in
// 32x32 MFMA accumulators (v_mfma_f32_32x32x16_f16, v_mfma_i32_32x32x32_i8,
// or four v_mfma_f32_32x32x2_f32 per K step for FP32 inputs).  The K tile is
// BKB bytes of every row (64 FP16, 128 INT8 or 32 FP32 elements at
// BKB = 128).  A is kept in LDS row-major (K contiguous) and read with
// ds_read_b128; B is kept in LDS as it sits in memory (N contiguous) and read
// with gfx950's transposing ds_read_b64_tr_b16 / ds_read_b64_tr_b8, which
// hands each lane the K-contiguous column slice the MFMA B operand wants
// (FP32, for which no transposing read exists, takes four ds_read_b32).
// The LDS images use 16-byte-chunk XOR swizzles chosen for gfx950's 64 banks
// (256 bytes per cycle), so that the fragment reads, the register drains and
// the DMA writes are free of bank conflicts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include "tdgemm.h"

namespace tdg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_ua __attribute__((ext_vector_type(4), aligned(1)));  // any byte alignment

#define TDG_LDS __attribute__((address_space(3)))
#define TDG_GLOBAL __attribute__((address_space(1)))

enum { DT_F16 = 0, DT_I8 = 1, DT_F32 = 2 };
enum { VAR_SINGLE = 1, VAR_REG = 2, VAR_DIRECT = 3 };

// Kernel arguments (passed by value).  Leading dimensions are in elements.
struct GemmArgs {
    const unsigned char *A;
    const unsigned char *B;
    unsigned char *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n;
    int k_tiles;  // ceil(K / BK); 0 when K == 0 (C is then zero-filled)
    int flags;    // TDG_DEBUG_* bits
    int k_rotate; // 1: tile row tm walks its K tiles from tm mod k_tiles
    // Split K: k_parts workgroups per C tile, part p taking K tiles
    // [p * k_per_part, min(k_tiles, (p + 1) * k_per_part)) and writing its
    // partial tile at C + p * part_stride bytes.  k_parts == 1: plain GEMM.
    int k_parts, k_per_part;
    int64_t part_stride;
};

// Compile-time geometry of one configuration.
template <int DT, int BM_, int BN_, int BKB_, int WM_, int WN_>
struct Geo {
    static constexpr int ES = DT == DT_F16 ? 2 : (DT == DT_I8 ? 1 : 4);  // input element bytes
    static constexpr int BM = BM_, BN = BN_, BKB = BKB_;
    static constexpr int BK = BKB / ES;  // K elements per tile
    static constexpr int WM = WM_, WN = WN_;
    static constexpr int NWAVES = WM * WN, NT = NWAVES * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    static constexpr int MI = WTM / 32, NI = WTN / 32;  // 32x32 MFMA blocks per wave
    static constexpr int KSTEPS = BKB / 32;             // MFMA K steps per tile (32 bytes each)
    // A image: BM rows of BKB bytes.
    static constexpr int A_CPR = BKB / 16;
    static constexpr int A_CHUNKS = BM * A_CPR;
    static constexpr int A_BYTES = BM * BKB;
    static constexpr int A_RP = 256 / BKB;  // A rows per 256-byte bank line
    // B image: BK rows (k) of BN*ES bytes.
    static constexpr int B_ROWB = BN * ES;
    static constexpr int B_CPR = B_ROWB / 16;
    static constexpr int B_CHUNKS = BK * B_CPR;
    static constexpr int B_BYTES = BK * B_ROWB;
    static constexpr int B_RP = B_ROWB >= 256 ? 1 : 256 / B_ROWB;
    // B fragments: FP16 / INT8 use gfx950's transposing 8-byte reads (two per
    // fragment); FP32 has no transposing read and takes four 4-byte reads.
    static constexpr bool TRB = DT != DT_F32;
    static constexpr int B_RD = TRB ? 2 : 4;  // LDS reads per B fragment
    // Transposed-read geometry: a 16-lane group reads TR_ROWS k-rows, LPR lanes
    // per row, EPL elements per lane; two adjacent groups read SEG_CH chunks.
    static constexpr int TR_ROWS = DT == DT_F16 ? 4 : 8;
    static constexpr int LPR = 16 / TR_ROWS;
    static constexpr int EPL = 8 / ES;
    static constexpr int SEG_CH = DT == DT_F16 ? 4 : 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int CA = A_CHUNKS / NT;  // A chunks per thread per tile
    static constexpr int CB = B_CHUNKS / NT;  // B chunks per thread per tile

    static_assert(BKB == 64 || BKB == 128, "K tile is 64 or 128 bytes per row");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "tile must split evenly over threads");
    static_assert((B_CPR & (B_CPR - 1)) == 0, "B row must be a power-of-two number of chunks");
    static_assert(!TRB || TR_ROWS >= B_RP, "B rows per bank line exceed the transposed-read group");
    static_assert(!TRB || SEG_CH * (TR_ROWS / B_RP) <= B_CPR, "B swizzle must stay inside a row");

    // Physical 16-byte chunk of logical chunk c in A row r.  Sixteen
    // consecutive rows read at one logical chunk land on 16 distinct
    // 16-byte bank slots of the 256-byte bank line.
    __device__ static __forceinline__ int swz_a(int r) { return (r / A_RP) % A_CPR; }
    // XOR applied to the chunk index of B row k: the TR_ROWS rows that one
    // transposed read touches, SEG_CH chunks each, land on distinct slots.
    // FP32 reads 4-byte words, half a wave per row: no swizzle needed.
    __device__ static __forceinline__ int swz_b(int k) {
        if constexpr (!TRB) return 0;
        return ((k / B_RP) % (TR_ROWS / B_RP)) * SEG_CH;
    }
};

// MFMA operand/accumulator types per dtype.
template <int DT>
struct Mfma;
// One K step (32 bytes of K per lane pair) is SUB MFMAs; mac_sub issues the
// e-th of them.
template <>
struct Mfma<DT_F16> {
    typedef f32x16 acc_t;
    typedef float out_t;
    static constexpr int SUB = 1;
    __device__ static __forceinline__ acc_t mac_sub(u32x4 a, u32x4 b, acc_t c, int) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    // Two transposed 8-byte reads give a lane its 8 K-consecutive halves.
    __device__ static __forceinline__ u32x4 read_b(const unsigned char *p0, const unsigned char *p1) {
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TDG_LDS i16x4 *)(p0));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TDG_LDS i16x4 *)(p1));
        i32x2 l2 = __builtin_bit_cast(i32x2, lo), h2 = __builtin_bit_cast(i32x2, hi);
        return u32x4{(uint32_t)l2[0], (uint32_t)l2[1], (uint32_t)h2[0], (uint32_t)h2[1]};
    }
};
template <>
struct Mfma<DT_I8> {
    typedef i32x16 acc_t;
    typedef int32_t out_t;
    static constexpr int SUB = 1;
    __device__ static __forceinline__ acc_t mac_sub(u32x4 a, u32x4 b, acc_t c, int) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                     __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
    // Two transposed 8-byte reads give a lane its 16 K-consecutive bytes.
    __device__ static __forceinline__ u32x4 read_b(const unsigned char *p0, const unsigned char *p1) {
        i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((TDG_LDS i32x2 *)(p0));
        i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((TDG_LDS i32x2 *)(p1));
        return u32x4{(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)hi[0], (uint32_t)hi[1]};
    }
};

// FP32: v_mfma_f32_32x32x2_f32 multiplies one binary32 of A (row l % 32) by
// one of B (column l % 32) per lane, at k = l / 32 of the instruction's two.
// A 16-byte A fragment holds a lane's four consecutive k (4h .. 4h+3 of the
// step's eight, h = l / 32), so the step is four MFMAs, the e-th taking
// element e of both fragments: it covers k = e and k = 4 + e.
template <>
struct Mfma<DT_F32> {
    typedef f32x16 acc_t;
    typedef float out_t;
    static constexpr int SUB = 4;
    // (The elements go through scalars: a bit cast applied directly to a
    // vector subscript reads element 0 whatever the index.)
    __device__ static __forceinline__ acc_t mac_sub(u32x4 a, u32x4 b, acc_t c, int e) {
        const uint32_t x = a[e], y = b[e];
        return __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, x),
                                                    __builtin_bit_cast(float, y), c, 0, 0, 0);
    }
    // Four 4-byte reads: rows k = 4h + e of the N-contiguous B image.
    __device__ static __forceinline__ u32x4 read_b4(const unsigned char *p0, const unsigned char *p1,
                                                    const unsigned char *p2, const unsigned char *p3) {
        return u32x4{*(const TDG_LDS uint32_t *)p0, *(const TDG_LDS uint32_t *)p1,
                     *(const TDG_LDS uint32_t *)p2, *(const TDG_LDS uint32_t *)p3};
    }
};

__device__ static __forceinline__ u32x4 lds_read16(const unsigned char *p) {
    return *(const TDG_LDS u32x4 *)(p);
}
__device__ static __forceinline__ void lds_write16(unsigned char *p, u32x4 v) {
    *(TDG_LDS u32x4 *)(p) = v;
}

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left unconstrained (gfx9
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ static __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Sixteen zero bytes: the source of every chunk that lies outside A or B on
// the bounds-checked paths, so that chunk lands in LDS as zeros while every
// lane still issues the same load or DMA instruction.
static __device__ __attribute__((aligned(16))) const uint32_t tdg_zero16[4] = {0u, 0u, 0u, 0u};

// Workgroup -> C tile.  Workgroups are dealt round-robin to the 8 XCDs, so
// when the tile count is a multiple of 8, workgroup b is renumbered so that
// each XCD receives a contiguous run of tile ids; the ids are then laid out in
// groups of GROUP_M tile rows, which gives every XCD a compact block of C
// tiles and lets its L2 reuse both A row panels and B column panels.
__device__ static __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
    constexpr int GROUP_M = 4;
    const int total = tiles_m * tiles_n;
    int id = bid;
    if ((total & 7) == 0) id = (bid & 7) * (total >> 3) + (bid >> 3);
    const int per_group = GROUP_M * tiles_n;
    const int group = id / per_group;
    const int first_m = group * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int r = id - group * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

// A 16-byte load at any byte alignment from global memory.  The source is
// chosen between an operand and the zero block, which would otherwise make it
// a generic (flat) pointer, and flat loads also count against the LDS wait
// counter.
__device__ static __forceinline__ u32x4 load16_global(const unsigned char *p) {
    return *(const __attribute__((address_space(1))) u32x4_ua *)p;
}

// One bounds-checked 16-byte chunk of a register-staged tile.  Rows outside
// the operand (A rows >= M, B rows k >= K) and, with ZERO_TAIL, elements at
// and beyond `valid` must read as zero: a k >= K would add to every sum.
// Without ZERO_TAIL (B's columns >= N) the bytes past `valid` may hold
// anything, because they only feed C columns that are never stored.
// Every chunk is ONE 16-byte load, at any byte alignment: the HSA runtime
// runs the chip in unaligned-access mode, and the compiler emits the same
// instruction for a 16-byte load through a byte-aligned pointer.  Choosing
// the source and correcting the loaded bytes are split, so that the loads of
// a whole tile issue back to back and the correction runs after they have
// landed, with no wait between them:
//   * whole chunk: the load from p, no correction;
//   * chunk outside the operand: the load from a zero block, no correction;
//   * partial chunk (a K or N tail) whose 16 bytes stay in the 4 KiB page of
//     p: the load from p, bytes past the valid ones zeroed afterwards when
//     ZERO_TAIL;
//   * partial chunk that would run past that page: the load of the 16 bytes
//     that end with the last valid byte (they start within p's page), shifted
//     down afterwards (and masked).
// GPU memory is mapped in pages of 4 KiB or more, so every byte loaded lies
// in a page that holds a valid byte.  `fix` returns the correction: 16 for
// none, else the valid byte count plus the downward shift in bits 8 and up.
template <int ES, bool ZERO_TAIL>
__device__ static __forceinline__ const unsigned char *chunk_source(const unsigned char *p, bool row_ok,
                                                                    int valid, uint32_t &fix) {
    constexpr int EPC = 16 / ES;
    const bool any = row_ok && valid > 0;
    const uint32_t nbytes = (uint32_t)valid * ES;  // < 16 when partial
    const bool tail = any && valid < EPC;
    const bool end_anchor = tail && ((uintptr_t)p & 4095) > 4096 - 16;
    const uint32_t shift = end_anchor ? 16u - nbytes : 0u;
    fix = tail && (ZERO_TAIL || end_anchor) ? (nbytes | shift << 8) : 16u;
    return !any ? (const unsigned char *)tdg_zero16 : p - shift;
}

__device__ static __forceinline__ u32x4 chunk_fixup(u32x4 v, uint32_t fix) {
    if (fix & 16u) return v;
    uint32_t w[4] = {v[0], v[1], v[2], v[3]};
    const uint32_t shift = fix >> 8;
    if (shift) {  // end-anchored chunk: move byte `shift` down to byte 0
        const uint32_t d[8] = {w[0], w[1], w[2], w[3], 0u, 0u, 0u, 0u};
        const uint32_t ds = shift >> 2, bs = shift & 3;
        // e[j] = d[ds + j], selected without indexing a register array
        uint32_t e[5];
#pragma unroll
        for (int j = 0; j < 5; j++) {
            const uint32_t x0 = d[j], x1 = d[j + 1], x2 = d[j + 2], x3 = d[j + 3];
            e[j] = ds == 0 ? x0 : ds == 1 ? x1 : ds == 2 ? x2 : x3;
        }
#pragma unroll
        for (int j = 0; j < 4; j++) w[j] = __builtin_amdgcn_alignbyte(e[j + 1], e[j], bs);  // bytes bs.. of e[j]:e[j+1]
    }
    // keep bytes [0, nbytes): word j keeps min(max(nbytes - 4j, 0), 4) bytes
    const int nbytes = (int)(fix & 15u);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int left = nbytes - 4 * j;
        const uint32_t keep = left >= 4 ? 32u : (left > 0 ? 8u * (uint32_t)left : 0u);
        w[j] &= (uint32_t)((1ull << keep) - 1ull);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

template <int DT, int BM, int BN, int BKB, int WM, int WN, int STAGES, int VAR, bool GUARD>
__global__ void __launch_bounds__(WM * WN * 64, 1) tdg_gemm_kernel(GemmArgs args) {
    typedef Geo<DT, BM, BN, BKB, WM, WN> G;
    typedef Mfma<DT> MM;
    typedef typename MM::acc_t acc_t;
    typedef typename MM::out_t out_t;
    static_assert(STAGES >= 1 && STAGES <= 8, "one to eight LDS buffers");
    static_assert(VAR == VAR_DIRECT || STAGES <= 2, "register staging holds one tile");
    static_assert(VAR != VAR_DIRECT || STAGES >= 2, "direct-to-LDS needs two or more buffers");
    static_assert(STAGES * G::STAGE_BYTES <= 160 * 1024, "LDS ring exceeds 160 KiB");
    static_assert(VAR != VAR_SINGLE || STAGES == 1, "the sequential baseline has one buffer");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGES * G::STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;

    int tm, tn;
    const int tile_id = (int)blockIdx.x / args.k_parts;
    const int part = (int)blockIdx.x - tile_id * args.k_parts;
    map_tile(tile_id, args.tiles_m, args.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kb = part * args.k_per_part;  // this workgroup's first K tile
    const int nt = min(args.k_tiles - kb, args.k_per_part);

    // Race screen: with the debug flag set, the whole LDS ring is filled with
    // 0xFF bytes before the first tile is requested.  A fragment read of a
    // buffer that the pipeline has not filled yet then sees NaN (FP16, FP32)
    // or -1 (INT8), and the result fails parity instead of passing on
    // whatever an earlier kernel left in LDS.
    if (args.flags & TDG_DEBUG_POISON_LDS) {
        for (int o = tid * 16; o < STAGES * G::STAGE_BYTES; o += G::NT * 16)
            lds_write16(smem + o, u32x4{~0u, ~0u, ~0u, ~0u});
        __syncthreads();
    }

    // Chunk i of this thread sits at LDS slot i*NT + tid of the A (or B)
    // image, i.e. image row i*RSTEP + tid/CPR and physical chunk tid % CPR.
    // The thread fetches the logical chunk that the swizzle puts there; the
    // swizzle of a row repeats every RSTEP rows, so one 32-bit per-lane
    // offset serves every i and every K tile, and the row/K advance goes into
    // a wave-uniform (SGPR) base address.  The same slots serve the register
    // drains and the LDS DMA, whose destinations are lane-contiguous.
    constexpr int A_RSTEP = G::NT / G::A_CPR;
    constexpr int B_RSTEP = G::NT / G::B_CPR;
    static_assert(A_RSTEP % (G::A_RP * G::A_CPR) == 0, "A swizzle must repeat every RSTEP rows");
    static_assert(!G::TRB || B_RSTEP % G::TR_ROWS == 0, "B swizzle must repeat every RSTEP rows");
    const int64_t lda_b = args.lda * G::ES, ldb_b = args.ldb * G::ES;
    const unsigned char *a_base = args.A + (int64_t)m0 * lda_b;
    const unsigned char *b_base = args.B + (int64_t)n0 * G::ES;
    const int a_r0 = tid / G::A_CPR, b_k0 = tid / G::B_CPR;
    const int a_c = (tid % G::A_CPR) ^ G::swz_a(a_r0);
    const int b_c = (tid % G::B_CPR) ^ G::swz_b(b_k0);
    const uint32_t a_voff = (uint32_t)(a_r0 * lda_b + a_c * 16);
    const uint32_t b_voff = (uint32_t)(b_k0 * ldb_b + b_c * 16);
    const uint32_t slot = (uint32_t)tid * 16u;
    const uint32_t smem_addr = (uint32_t)(uintptr_t)(TDG_LDS unsigned char *)smem;

    // Per-lane LDS read offsets of the MFMA fragments (within one stage).
    uint32_t a_roff[G::KSTEPS];
    {
        const int r = wm * G::WTM + (lane & 31);
#pragma unroll
        for (int s = 0; s < G::KSTEPS; s++)
            a_roff[s] = (uint32_t)(r * G::BKB + (((2 * s + (lane >> 5)) ^ G::swz_a(r)) * 16));
    }
    // FP32 B reads need no swizzle, so every read address is one per-lane
    // base plus a constant (folded into the instruction's offset field).
    const uint32_t b_roff32 = (uint32_t)(G::A_BYTES + ((lane >> 5) * 4) * G::B_ROWB +
                                         (wn * G::WTN + (lane & 31)) * G::ES);
    // Transposed B reads (FP16, INT8): the swizzle of a k-row repeats every
    // TR_ROWS rows, and K steps and the reads within a step advance k by
    // multiples of TR_ROWS, so every read of column block ni is one per-lane
    // offset (step 0, read 0) plus a compile-time constant that goes into the
    // instruction's offset field.  With two or more column blocks per wave
    // that saves registers: one per block instead of one per (step, read,
    // block), 12 fewer in the 8-wave INT8 256 x 256 kernel, which gave the
    // bounds-checked kernels room for the 3-step read distance.  With one
    // block (the 64 x 64 tile) the per-step offsets are kept: folded, the
    // skinny product ran 1.3% slower (and FP16 1024^3 2% faster).
    constexpr int B_KS = 32 / G::ES;   // k per MFMA step
    constexpr int B_KR = G::TR_ROWS;   // k per transposed read
    static_assert(!G::TRB || (B_KS % G::TR_ROWS == 0 && (B_KS / 2) % G::TR_ROWS == 0),
                  "B swizzle must repeat across K steps");
    constexpr bool B_FOLD = G::NI >= 2;
    constexpr int B_S = G::TRB && !B_FOLD ? G::KSTEPS : 1, B_H = G::TRB && !B_FOLD ? G::B_RD : 1;
    uint32_t b_roff[B_S][B_H][G::TRB ? G::NI : 1];
    if constexpr (G::TRB) {
#pragma unroll
        for (int s = 0; s < B_S; s++)
#pragma unroll
            for (int h = 0; h < B_H; h++) {
                // k-row group h of the lane's half (lane / 32) of step s
                const int k = s * B_KS + (lane >> 5) * (B_KS / 2) + h * B_KR + (lane & 15) / G::LPR;
#pragma unroll
                for (int ni = 0; ni < G::NI; ni++) {
                    const int n = wn * G::WTN + ni * 32 + ((lane >> 4) & 1) * 16 + (lane % G::LPR) * G::EPL;
                    const int byte = n * G::ES;
                    b_roff[s][h][ni] = (uint32_t)(G::A_BYTES + k * G::B_ROWB +
                                                  (((byte >> 4) ^ G::swz_b(k)) << 4) + (byte & 15));
                }
            }
    }
    // LDS offset of read h of K step s of column block ni.
    auto b_off = [&](int s, int h, int ni) -> uint32_t {
        if constexpr (B_FOLD) return b_roff[0][0][ni] + (uint32_t)((s * B_KS + h * B_KR) * G::B_ROWB);
        else return b_roff[s][h][ni];
    };

    acc_t acc[G::MI][G::NI];
#pragma unroll
    for (int mi = 0; mi < G::MI; mi++)
#pragma unroll
        for (int ni = 0; ni < G::NI; ni++) acc[mi][ni] = acc_t{};

    // ---- building blocks ---------------------------------------------------
    u32x4 ra[G::CA], rb[G::CB];  // register staging (SINGLE / REG)
    uint32_t fix_a[G::CA], fix_b[G::CB];  // their corrections (GUARD)

    // K-tile rotation (k_rotate, chosen on the host when all of B fits in
    // half an XCD's L2): tile row tm starts its K walk at tile tm mod nt and
    // wraps.  Workgroups of one tile row share A panels and stay in lock
    // step; B is read from L2 in any order.  What changes is A's pattern in
    // HBM: without the rotation every workgroup reads the same K columns of
    // its rows at once, and with a row stride that is a multiple of the HBM
    // channel interleave those reads land on a few channels.  `kt` below is
    // the position in the walk over this workgroup's nt tiles (its K part);
    // phys() is the K tile it loads.  Every loop form uses the same walk, so
    // their results stay bitwise identical.
    const int krot = args.k_rotate && nt > 0 ? tm % nt : 0;
    auto phys = [&](int kt) { return kb + (kt + krot >= nt ? kt + krot - nt : kt + krot); };
    auto a_ptr = [&](int kt, int i) {
        return a_base + (int64_t)kt * G::BKB + (int64_t)(i * A_RSTEP) * lda_b;
    };
    auto b_ptr = [&](int kt, int i) {
        return b_base + (int64_t)(kt * G::BK + i * B_RSTEP) * ldb_b;
    };
    auto load_regs = [&](int kt) {
        kt = phys(kt);
        if (!GUARD) {
#pragma unroll
            for (int i = 0; i < G::CA; i++) ra[i] = *(const u32x4 *)(a_ptr(kt, i) + a_voff);
#pragma unroll
            for (int i = 0; i < G::CB; i++) rb[i] = *(const u32x4 *)(b_ptr(kt, i) + b_voff);
        } else {
            // Only the last K tile (when K is not a whole number of tiles)
            // and the M or N edge tiles need the checks; the test is uniform
            // over the workgroup, so interior tiles take plain sources.  All
            // sources are chosen before the first load issues: address work
            // between loads can make the compiler wait for the loads already
            // in flight.
            const int kbase = kt * G::BK;
            constexpr int EPC = 16 / G::ES;
            const bool k_inside = kbase + G::BK <= args.K;
            const unsigned char *src_a[G::CA], *src_b[G::CB];
            if (k_inside && m0 + G::BM <= args.M) {
#pragma unroll
                for (int i = 0; i < G::CA; i++) {
                    src_a[i] = a_ptr(kt, i) + a_voff;
                    fix_a[i] = 16u;
                }
            } else {
#pragma unroll
                for (int i = 0; i < G::CA; i++) {
                    const bool row_ok = m0 + i * A_RSTEP + a_r0 < args.M;
                    const int valid = args.K - (kbase + a_c * EPC);
                    src_a[i] = chunk_source<G::ES, true>(a_ptr(kt, i) + a_voff, row_ok, valid, fix_a[i]);
                }
            }
            if (k_inside && n0 + G::BN <= args.N) {
#pragma unroll
                for (int i = 0; i < G::CB; i++) {
                    src_b[i] = b_ptr(kt, i) + b_voff;
                    fix_b[i] = 16u;
                }
            } else {
#pragma unroll
                for (int i = 0; i < G::CB; i++) {
                    const bool row_ok = kbase + i * B_RSTEP + b_k0 < args.K;
                    const int valid = args.N - (n0 + b_c * EPC);
                    src_b[i] = chunk_source<G::ES, false>(b_ptr(kt, i) + b_voff, row_ok, valid, fix_b[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < G::CA; i++) ra[i] = load16_global(src_a[i]);
#pragma unroll
            for (int i = 0; i < G::CB; i++) rb[i] = load16_global(src_b[i]);
        }
    };
    // One chunk of an unchecked register load (d: A chunks first, then B).
    auto load_one = [&](int kt, int d) __attribute__((always_inline)) {
        kt = phys(kt);
        if (d < G::CA) ra[d] = *(const u32x4 *)(a_ptr(kt, d) + a_voff);
        else rb[d - G::CA] = *(const u32x4 *)(b_ptr(kt, d - G::CA) + b_voff);
    };
    // Drain staged chunk d (A chunks first, then B) into the buffer at st.
    auto store_one = [&](unsigned char *st, int d) {
        if (d < G::CA) {
            lds_write16(st + slot + d * G::NT * 16, GUARD ? chunk_fixup(ra[d], fix_a[d]) : ra[d]);
        } else {
            const int i = d - G::CA;
            lds_write16(st + G::A_BYTES + slot + i * G::NT * 16,
                        GUARD ? chunk_fixup(rb[i], fix_b[i]) : rb[i]);
        }
    };
    auto store_regs = [&](unsigned char *st) {
#pragma unroll
        for (int d = 0; d < G::CA + G::CB; d++) store_one(st, d);
    };
    // LDS DMA: each lane's 16 bytes land at M0 + 16 * lane.  Issued from
    // inline assembly so that the compiler does not guard the other buffer's
    // LDS reads with a wait on these copies; completion is awaited
    // explicitly (vmcnt) before the barrier that publishes the tile.
    // Bounds-checked DMA (GUARD, with the `checked` tag set): chunks sit on a
    // 16-byte grid from each row's first byte, at any alignment (the DMA
    // reads 16 bytes from any byte address).  A chunk that starts outside its
    // matrix (A row >= M, k >= K; B row k >= K, column >= N) is fetched from
    // the zero block instead; one that starts inside is fetched whole, also
    // when K or N ends inside it.  Its bytes past the row's end then belong
    // to the next row, except at the end of the last row, where the host
    // runs this loop only when the chunk holding the operand's last byte
    // stays in that byte's 4 KiB page.  The source is then a per-lane 64-bit
    // address.  B columns >= N and A rows >= M only
    // feed C elements that are never stored; k >= K must be zero, which the
    // zero block gives for whole chunks and clear_k_tail for the one A chunk
    // per row that K splits.  A bounds-checked kernel issues the plain form (wave-uniform
    // base, 32-bit lane offset) for every K tile known to lie wholly inside
    // the operands, so only edge workgroups and the K tail pay for checks.
    constexpr int EPC = 16 / G::ES;
    uint32_t a_rows_ok = 0;
    if constexpr (GUARD) {
#pragma unroll
        for (int i = 0; i < G::CA; i++)
            if (m0 + i * A_RSTEP + a_r0 < args.M) a_rows_ok |= 1u << i;
    }
    const bool b_col_ok = n0 + b_c * EPC < args.N;
    const int a_kc = a_c * EPC;  // first k of this thread's A chunk within a tile
    const uint64_t zero_addr = (uint64_t)(uintptr_t)tdg_zero16;
    auto issue_direct_one = [&](uint32_t st_off, int kt, int d, auto checked) __attribute__((always_inline)) {
        kt = phys(kt);
        const uint32_t wbase = smem_addr + st_off + (uint32_t)wave * 1024u;
        if constexpr (GUARD && decltype(checked)::value) {
            // Branch-free: the address is formed whether or not the chunk is
            // inside, and a select (two v_cndmask) swaps in the zero block;
            // the tests combine with bitwise & so that no short-circuit
            // turns them into divergent branches around every DMA.
            const int k_lim = args.K - kt * G::BK;  // k of this tile inside K
            uint64_t src;
            uint32_t m0v;
            if (d < G::CA) {
                const uint64_t p = (uint64_t)(uintptr_t)(a_ptr(kt, d) + a_voff);
                const bool ok = (bool)((a_rows_ok >> d) & 1u) & (a_kc < k_lim);
                src = ok ? p : zero_addr;
                m0v = wbase + (uint32_t)(d * G::NT * 16);
            } else {
                const int i = d - G::CA;
                const uint64_t p = (uint64_t)(uintptr_t)(b_ptr(kt, i) + b_voff);
                const bool ok = b_col_ok & (i * B_RSTEP + b_k0 < k_lim);
                src = ok ? p : zero_addr;
                m0v = wbase + (uint32_t)(G::A_BYTES + i * G::NT * 16);
            }
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0v) : "memory");
            return;
        }
        // the tile index is wave-uniform; the bounds-checked kernels' uniformity
        // analysis does not see it, and the base address must be scalar
        if constexpr (GUARD) kt = __builtin_amdgcn_readfirstlane(kt);
        if (d < G::CA) {
            const uint32_t m0v = wbase + (uint32_t)(d * G::NT * 16);
            asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(a_voff), "s"(a_ptr(kt, d)),
                         "{m0}"(m0v)
                         : "memory");
        } else {
            const int i = d - G::CA;
            const uint32_t m0v = wbase + (uint32_t)(G::A_BYTES + i * G::NT * 16);
            asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(b_voff), "s"(b_ptr(kt, i)),
                         "{m0}"(m0v)
                         : "memory");
        }
    };
    auto issue_direct = [&](uint32_t st_off, int kt, auto checked) __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < G::CA + G::CB; d++) issue_direct_one(st_off, kt, d, checked);
    };

    // MFMA tile micro-kernel over one LDS buffer.  The fragments of K step
    // s + FD are requested from LDS while the MFMAs of step s issue (FD
    // register sets ahead), so the LDS latency hides behind matrix work; the
    // scheduling barriers keep the compiler from sinking the reads back next
    // to their first use.  When the reads run past the tile, the
    // loop-specific `boundary` runs first: it publishes the next tile, whose
    // first fragments are then read into their sets, so the tile change
    // costs no exposed LDS latency either.
    static_assert(G::KSTEPS % 2 == 0, "fragment set parity must repeat per tile");
    // Fragment read distance: when a tile has 4 K steps, the direct-to-LDS
    // loop keeps one register set per step and reads 3 steps ahead, else 1
    // (two sets); the register-prefetch loop has no room for more sets beside
    // its staging.  Reading 3 steps ahead put the tile boundary, with its
    // wait and barrier, one step earlier, and together with the copies spread
    // over two steps (below) made the 256 x 256 tiles about 1.5% faster (FP16
    // and INT8 4096^3).
    constexpr int FD = (VAR == VAR_DIRECT && G::KSTEPS == 4) ? 3 : 1;
    constexpr int NSETS = FD == 1 ? 2 : G::KSTEPS;
    static_assert(FD == 1 || NSETS == G::KSTEPS, "set index must equal the step index");
    u32x4 fa[NSETS][G::MI], fb[NSETS][G::NI];
    auto read_bfrag = [&](const unsigned char *st, int s, int ni) -> u32x4 {
        if constexpr (G::TRB) {
            return MM::read_b(st + b_off(s, 0, ni), st + b_off(s, 1, ni));
        } else {
            // rows k = 8 s + 4 (l / 32) + h, h = 0..3; column block ni
            const unsigned char *p = st + b_roff32 + (s * 8) * G::B_ROWB + ni * 32 * G::ES;
            return MM::read_b4(p, p + G::B_ROWB, p + 2 * G::B_ROWB, p + 3 * G::B_ROWB);
        }
    };
    auto read_frags = [&](const unsigned char *st, int s, int set) {
#pragma unroll
        for (int mi = 0; mi < G::MI; mi++) fa[set][mi] = lds_read16(st + a_roff[s] + mi * 32 * G::BKB);
#pragma unroll
        for (int ni = 0; ni < G::NI; ni++) fb[set][ni] = read_bfrag(st, s, ni);
    };
    // One K step's MFMAs with the fragment reads of a later step (read
    // units: MI A reads, then NI pairs of transposed B reads) and, from the
    // tile boundary on, DMA instructions [dma_lo, dma_hi) of a later tile
    // spread between them: after MFMA m come the units and DMAs whose even
    // share falls on m.
    // Vector-memory and LDS instructions issue in order per wave, so a burst
    // of them from every wave at once queues and holds back each wave's next
    // MFMAs; spread out, each one issues into an idle queue while the MFMA
    // pipe stays busy.
    // With SUB > 1 (FP32) the step's MFMAs go round-robin over the
    // accumulators, so dependent MFMAs are NM instructions apart.
    // Register-prefetch loop with two buffers on unchecked whole tiles: the
    // drain of tile t+1 runs in tile t's next-to-last step, and the tile
    // whose global loads are issued chunk by chunk right after it, as each
    // staging register is freed (EARLY_REG; see the K loop).
    constexpr bool EARLY_REG = VAR == VAR_REG && STAGES == 2 && G::KSTEPS >= 4 && !GUARD;
    int reg_ahead = 0;
    auto step = [&](int cset, const unsigned char *rst, int rstep, int rset, bool reads,
                    uint32_t dma_st, int dma_kt, int dma_lo, int dma_hi, unsigned char *wst, bool drain,
                    auto checked) {
        constexpr int NM = G::MI * G::NI, NR = G::MI + G::NI, ND = G::CA + G::CB;
        constexpr int NMF = NM * MM::SUB;  // MFMA issue slots in the step
#pragma unroll
        for (int t = 0; t < NMF; t++) {
            const int m = t % NM, e = t / NM;
            acc[m / G::NI][m % G::NI] =
                MM::mac_sub(fa[cset][m / G::NI], fb[cset][m % G::NI], acc[m / G::NI][m % G::NI], e);
            __builtin_amdgcn_sched_barrier(0);
            if (reads) {
#pragma unroll
                for (int u = (t * NR + NMF - 1) / NMF; u < ((t + 1) * NR + NMF - 1) / NMF; u++) {
                    if (u < G::MI) {
                        fa[rset][u] = lds_read16(rst + a_roff[rstep] + u * 32 * G::BKB);
                    } else {
                        fb[rset][u - G::MI] = read_bfrag(rst, rstep, u - G::MI);
                    }
                }
            }
            if (dma_hi > dma_lo) {
                const int nd = dma_hi - dma_lo;
#pragma unroll
                for (int d = (t * nd + NMF - 1) / NMF; d < ((t + 1) * nd + NMF - 1) / NMF; d++)
                    issue_direct_one(dma_st, dma_kt, dma_lo + d, checked);
            }
            if constexpr (EARLY_REG) {
                if (drain) {
#pragma unroll
                    for (int d = (t * ND + NMF - 1) / NMF; d < ((t + 1) * ND + NMF - 1) / NMF; d++) {
                        store_one(wst, d);
                        load_one(reg_ahead, d);  // its staging register is free now
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto set_of = [&](int s) { return NSETS == 2 ? (s & 1) : s; };
    // Reads the first FD steps of the tile in buffer st.
    auto read_first = [&](const unsigned char *st) {
#pragma unroll
        for (int s = 0; s < FD; s++) read_frags(st, s, set_of(s));
    };
    // Computes the tile in buffer st, whose first FD steps are already in
    // registers.  `boundary` runs when the reads run past this tile: it
    // publishes the next tile (when there is one) and returns the buffer the
    // reads continue in -- for the last tile a buffer whose contents are
    // never used, so the step is the same straight-line code every time.
    // For the direct-to-LDS loop it also names the tile whose DMA is
    // interleaved with the MFMAs of the step it runs in.
    // For the register-prefetch loop with two buffers, `early_st` names the
    // other buffer when the next tile is staged: its drain is spread over
    // the MFMAs of the next-to-last step (the loads were issued a whole
    // tile earlier, so they have landed by then), and the tile boundary
    // keeps only the barrier that publishes it.  Measured 1-2% faster on
    // interior tiles; the bounds-checked form keeps the drain at the
    // boundary, where its byte fix-ups cost less than between the MFMAs.
    // The copies of a later tile go out over SPREAD steps from the boundary
    // on: two in the direct-to-LDS loop with a read distance of 2 or more,
    // which halves the vector-memory instructions per step.  Every copy of
    // the tile is issued before the next boundary, so the vmcnt counts do
    // not change.
    constexpr int SPREAD = VAR == VAR_DIRECT && FD >= 2 ? 2 : 1;
    constexpr int ND_ALL = G::CA + G::CB;
    int dma_tile = 0;
    uint32_t dma_off = 0;
    unsigned char *early_st = nullptr;
    auto compute_tile = [&](const unsigned char *st, auto &&boundary, auto checked) {
        const unsigned char *next = st;
#pragma unroll
        for (int s = 0; s < G::KSTEPS; s++) {
            const int r = s + FD;  // step whose fragments are read now
            if (r == G::KSTEPS) next = boundary();
            const unsigned char *rst = r < G::KSTEPS ? st : next;
            const int rstep = r < G::KSTEPS ? r : r - G::KSTEPS;
            // the copies of a later tile: DMA instructions [lo, hi) of the step
            const int part = VAR == VAR_DIRECT && r >= G::KSTEPS && r < G::KSTEPS + SPREAD ? r - G::KSTEPS : -1;
            const int lo = part < 0 ? 0 : part * ND_ALL / SPREAD;
            const int hi = part < 0 ? 0 : (part + 1) * ND_ALL / SPREAD;
            step(set_of(s), rst, rstep, set_of(rstep), true, dma_off, dma_tile, lo, hi, early_st,
                 EARLY_REG && s == G::KSTEPS - 2, checked);
        }
    };
    using unchecked_t = std::false_type;
    using checked_t = std::true_type;
    auto buf = [&](int t) { return smem + (t % STAGES) * G::STAGE_BYTES; };

    // ---- K loop ------------------------------------------------------------
    // Every form has the pages' three parts: a prologue that stages tile 0
    // (and, pipelined, the tiles after it), a main loop that computes tile t
    // while later tiles load, and an epilogue in which the last tiles are
    // computed with nothing left to load ("Pipeline GPU Kernel", Step 3).
    if (nt > 0) {
        if constexpr (VAR == VAR_SINGLE) {
            // Sequential: load -> barrier -> compute -> barrier, every tile.
            for (int t = 0; t < nt; t++) {
                load_regs(t);
                if (t > 0) __syncthreads();  // everyone finished computing on the buffer
                store_regs(smem);
                __syncthreads();
                read_first(smem);
                compute_tile(smem, [&]() -> const unsigned char * { return smem; }, unchecked_t{});
            }
        } else if constexpr (VAR == VAR_REG) {
            // Main loop + epilogue: tile t+1 is in registers (global loads in
            // flight) while tile t is computed; the registers are drained into
            // buffer (t+1) % STAGES at the tile boundary.
            // With two buffers on unchecked whole tiles (EARLY_REG), the drain
            // of tile t+1 is spread over the MFMAs of tile t's next-to-last
            // step, and each staging register, once drained, at once receives
            // its chunk of tile t+2: the loads then have a whole tile of MFMAs
            // to land in, not just the steps before the drain.  The drain and
            // the loads run in every tile, so that the compiler can count the
            // loads in flight (a conditional load makes it wait for all of
            // them): past the end, the last tile is loaded again and drained
            // into the buffer just freed, which is never read again.
            constexpr bool EARLY = EARLY_REG;
            // Prologue: tile 0 into buffer 0 (and, EARLY, tile 1 into registers).
            load_regs(0);
            store_regs(smem);
            __syncthreads();
            if (EARLY) load_regs(min(1, nt - 1));
            read_first(smem);
            for (int t = 0; t < nt; t++) {
                if (!EARLY && t + 1 < nt) load_regs(t + 1);
                __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
                early_st = EARLY ? buf(t + 1) : nullptr;
                reg_ahead = min(t + 2, nt - 1);
                compute_tile(buf(t), [&]() -> const unsigned char * {
                    if (t + 1 < nt) {
                        if (!EARLY) {
                            if (STAGES == 1) __syncthreads();  // all reads of the buffer done
                            store_regs(buf(t + 1));
                        }
                        __syncthreads();  // drained tile visible to every wave
                    }
                    return buf(t + 1);
                }, unchecked_t{});
            }
        } else {
            // Ring of STAGES buffers, AHEAD = STAGES - 1 tiles in flight.
            // Tile t lives in buffer t % STAGES; it is waited for with a
            // partial vmcnt (the AHEAD - 1 younger tiles stay in flight),
            // published by the barrier, which also certifies that every wave
            // has finished reading tile t - 1, whose buffer then receives tile
            // t + AHEAD.  Every boundary issues exactly one tile: past the last
            // tile it loads the last tile again into the buffer just freed,
            // which is never read again, so the number of younger groups at
            // every wait is AHEAD - 1 and the wait count is a constant.
            constexpr int AHEAD = STAGES - 1;
            constexpr int IPT = G::CA + G::CB;  // DMA instructions per wave per tile
            static_assert(AHEAD * IPT <= 63, "vmcnt holds at most 63");
            auto stage_off = [&](int t) { return (uint32_t)((t % STAGES) * G::STAGE_BYTES); };
            auto src_tile = [&](int t) { return t < nt ? t : nt - 1; };
            // Walk positions from `w_chk` on take the bounds-checked DMA: all
            // of them in an edge workgroup (its tile crosses M or N), else
            // those from the partial last K tile on (K not a whole number of
            // tiles), else none.  Positions after a rotated walk wraps past
            // the partial tile are whole again but stay checked.
            int w_chk = nt;
            if constexpr (GUARD) {
                const int last = args.k_tiles - 1;  // the only tile that can be partial
                if (m0 + BM > args.M || n0 + BN > args.N) {
                    w_chk = 0;
                } else if (args.K % G::BK != 0 && last >= kb && last < kb + nt) {
                    const int w = last - kb - krot;
                    w_chk = w < 0 ? w + nt : w;
                }
            }
            auto issue_pos = [&](uint32_t off, int w) __attribute__((always_inline)) {
                if (w >= w_chk) issue_direct(off, w, checked_t{});
                else issue_direct(off, w, unchecked_t{});
            };
            // A K that splits a 16-byte chunk: the last K tile's straddling
            // chunk of every A row is fetched whole (see the bounds-checked
            // DMA above), so its bytes at k >= K hold whatever follows in
            // memory.  Once that tile has landed and
            // been published, each row's chunk is cleared from byte
            // (K - k0) * sizeof(T) % 16 on, and a second barrier publishes
            // the cleared tile before any fragment is read.  (B needs no
            // such step: B rows k >= K come from the zero block, and B's
            // bytes past an N that splits a chunk only feed C columns that
            // are never stored.)
            int w_part = -1;   // walk position of the tile with the straddling chunk
            int kr_part = 0;   // valid k of that tile
            if constexpr (GUARD) {
                const int last = args.k_tiles - 1;
                if (((args.K * G::ES) & 15) != 0 && last >= kb && last < kb + nt) {
                    const int w = last - kb - krot;
                    w_part = w < 0 ? w + nt : w;
                    kr_part = args.K - last * G::BK;
                }
            }
            auto clear_k_tail = [&](int w) __attribute__((always_inline)) {
                if (!GUARD || w != w_part) return;
                if (tid < BM) {
                    const int lc = (kr_part * G::ES) >> 4;          // the straddling chunk
                    const uint32_t keep = (uint32_t)((kr_part * G::ES) & 15);  // its valid bytes
                    unsigned char *p = smem + (w % STAGES) * G::STAGE_BYTES + tid * G::BKB +
                                       ((lc ^ G::swz_a(tid)) << 4);
                    const u32x4 v = lds_read16(p);
                    uint32_t w4[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int left = (int)keep - 4 * j;
                        const uint32_t bits = left >= 4 ? 32u : (left > 0 ? 8u * (uint32_t)left : 0u);
                        w4[j] &= (uint32_t)((1ull << bits) - 1ull);
                    }
                    lds_write16(p, u32x4{w4[0], w4[1], w4[2], w4[3]});
                }
                __syncthreads();
            };
            // Prologue: tiles 0 .. AHEAD issued into the STAGES buffers, all
            // free at the start, then tile 0 awaited (the AHEAD younger tiles
            // stay in flight) and published: tile AHEAD loads during tile 0's
            // wait as well as its compute.
#pragma unroll
            for (int p = 0; p <= AHEAD; p++) issue_pos(stage_off(p), src_tile(p));
            wait_vmcnt<AHEAD * IPT>();
            __syncthreads();
            clear_k_tail(0);
            read_first(buf(0));
            // Main loop and epilogue (from tile nt - AHEAD on, the issued
            // loads are the harmless repeats).  The DMA interleaved with tile
            // t is for walk position min(t + 1 + AHEAD, nt - 1), which grows
            // with t, so the loop runs in two parts: plain DMA up to t_chk,
            // checked DMA from there (one copy of the loop in an unguarded
            // kernel).
            auto run_tiles = [&](int t0, int t1, auto checked) __attribute__((always_inline)) {
                for (int t = t0; t < t1; t++) {
                    compute_tile(buf(t), [&]() -> const unsigned char * {
                        if (t + 1 < nt) {
                            wait_vmcnt<(AHEAD - 1) * IPT>();  // tile t+1 landed
                            __syncthreads();
                            clear_k_tail(t + 1);
                            dma_tile = src_tile(t + 1 + AHEAD);  // issued between this step's MFMAs
                            dma_off = stage_off(t + 1 + AHEAD);
                        } else {
                            // last tile: no barrier; the repeat load goes to
                            // the buffer of tile t - 1, which every wave has
                            // finished reading (certified by the previous
                            // barrier) and which is never read again
                            dma_tile = nt - 1;
                            dma_off = stage_off(t - 1 + STAGES);
                        }
                        return buf(t + 1);
                    }, checked);
                }
            };
            if constexpr (GUARD) {
                const int t_chk = w_chk >= nt ? nt : max(0, w_chk - 1 - AHEAD);
                run_tiles(0, t_chk, unchecked_t{});
                run_tiles(t_chk, nt, checked_t{});
            } else {
                run_tiles(0, nt, unchecked_t{});
            }
            // Drain the repeat loads before the workgroup ends: LDS written by
            // a DMA still in flight could otherwise land in the next
            // workgroup's allocation.
            wait_vmcnt<0>();
        }
    }

    // ---- C write-back: 32x32 accumulator layout -> row-major C -------------
    // lane l of block (mi, ni) holds rows 8*(v/4) + 4*(l/32) + v%4, column l%32.
    // Every tile load has landed by now; saying so with a counted wait keeps
    // the compiler from guarding the stores' address registers (once tile
    // load destinations) with waits on the stores themselves.
    // One store instruction writes 128 contiguous bytes of each of two rows.
    // When C's rows start on 128-byte lines, those are whole lines and the
    // stores are non-temporal: C is written once and not read back by this
    // kernel, and streaming it past the L2 keeps the A and B lines that
    // workgroups still running read (FP16 / INT8 4096^3: about 1% faster).
    // Otherwise every 128 bytes straddle two lines, and non-temporal partial
    // lines reach memory as separate partial writes (INT8 4095^3 with
    // ldc = 4095: 1427 TOP/s against 2086 with plain stores); plain stores
    // let the L2 merge them into whole lines first.
    // A bounds-checked kernel stores interior tiles without the per-element
    // test (a uniform branch), so only edge tiles pay for the masking.
    wait_vmcnt<0>();
    out_t *C = (out_t *)(args.C + (int64_t)part * args.part_stride);
    const bool lines = ((uintptr_t)C & 127) == 0 && ((args.ldc * (int64_t)sizeof(out_t)) & 127) == 0;
    const int col_l = lane & 31, rq = (lane >> 5) * 4;
    auto store_all = [&](auto masked, auto streaming) __attribute__((always_inline)) {
#pragma unroll
        for (int mi = 0; mi < G::MI; mi++)
#pragma unroll
            for (int ni = 0; ni < G::NI; ni++) {
                const int col = n0 + wn * G::WTN + ni * 32 + col_l;
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int row = m0 + wm * G::WTM + mi * 32 + (v >> 2) * 8 + rq + (v & 3);
                    if (!decltype(masked)::value || (row < args.M && col < args.N)) {
                        out_t *p = &C[(int64_t)row * args.ldc + col];
                        if constexpr (decltype(streaming)::value)
                            __builtin_nontemporal_store(acc[mi][ni][v], p);
                        else
                            *p = acc[mi][ni][v];
                    }
                }
            }
    };
    // (The bounds-checked kernels always store plainly: one store form fewer
    // keeps their register use down, and on the ragged shapes they serve
    // plain stores measured as fast: FP16 / INT8 4000^3 1157 / 2089 against
    // 1157 / 2052.)
    if constexpr (!GUARD) {
        if (lines)
            store_all(std::false_type{}, std::true_type{});
        else
            store_all(std::false_type{}, std::false_type{});
    } else if (m0 + BM <= args.M && n0 + BN <= args.N) {
        store_all(std::false_type{}, std::false_type{});
    } else {
        store_all(std::true_type{}, std::false_type{});
    }
}

}  // namespace tdg
