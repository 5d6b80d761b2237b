// tdg_move.hip -- the copy / transpose ladder on HBM ("fixing GPU kernels by
// hand", the four-step transpose exercise), built for gfx950.
//
// A rows x cols matrix of 32-bit elements is copied (out[i][j] = in[i][j],
// the bandwidth upper bound) or transposed (out[j][i] = in[i][j]).  Nothing is
// computed; every form moves the same bytes and differs only in how it touches
// memory.  The page's ladder, on 32-wide warps and 32 banks, becomes on
// gfx950's 64-wide waves and 64 LDS banks of 4 bytes:
//   NAIVE         coalesced reads, writes strided by the output row length:
//                 each lane of a wave writes 4 bytes to a different row.
//   LDS           through a 64 x 64 tile in LDS; the tile is written by rows
//                 and read by columns, and a column of a 64-word-wide tile
//                 sits in one bank: every read is a 64-way bank conflict.
//   LDS_PADDED    the page's fix: one extra word per tile row, so column
//                 element r sits in bank (r + c) mod 64 -- conflict-free.
//   LDS_SWIZZLED  the same effect without the extra word: element (r, c) is
//                 stored at column c XOR r of row r.
//   VEC           gfx950's form: 16-byte loads and stores on both sides of
//                 the tile (a lane moves four elements per access); the tile
//                 is stored already transposed with a 4-word XOR swizzle, so
//                 the 16-byte LDS reads are conflict-free.
// The copy marks its global accesses non-temporal: nothing is read twice, and
// on a 1 GiB copy that measured 4-7% more bandwidth.  (The same hint made
// VEC slower, at both sizes measured, so VEC keeps ordinary accesses.)
// Tiles are 64 x 64 elements, one workgroup of 256 threads (4 waves) each;
// the transposes take them in diagonal order (tile_origin).
// Partial tiles at the matrix edges take element-wise, bounds-checked paths;
// VEC runs its vector path on whole tiles of 16-byte aligned operands and
// falls back to the swizzled element-wise path elsewhere.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "tdg_internal.h"
#include "tdgemm.h"

namespace {

constexpr int TILE = 64;
constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;
constexpr int ROWS_PER_PASS = WAVES;   // element-wise paths: one row per wave per pass
constexpr int CHUNKS_PER_ROW = TILE / 4;  // 16-byte chunks in a tile row
constexpr int VEC_ROWS_PER_PASS = THREADS / CHUNKS_PER_ROW;  // 16

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct MoveArgs {
    const uint32_t *in;
    uint32_t *out;
    int64_t ldi, ldo;
    int rows, cols;
    int tiles_c;  // tiles along a row of the input
    int tiles_r;  // tiles along a column of the input
    int vec_ok;   // 16-byte aligned bases and leading dimensions
    int diagonal; // 1: diagonal tile order (the transposes)
};

// Workgroup -> tile.  The copy walks the tiles row by row.  A transpose walks
// them diagonally: workgroup t takes tile column t mod tiles_c and tile row
// (t / tiles_c + t mod tiles_c) mod tiles_r, a bijection.  Row by row,
// workgroups running side by side would write output tiles that differ only
// in their output rows; with a power-of-two row length those addresses are a
// multiple of the HBM channel interleave apart and crowd a few channels.
// Diagonally, neighbours write at neighbouring output column offsets and read
// at neighbouring input column offsets, so both spread over the channels.
__device__ __forceinline__ void tile_origin(const MoveArgs &a, int &r0, int &c0) {
    const int t = blockIdx.x;
    const int q = t / a.tiles_c, tx = t % a.tiles_c;
    const int ty = a.diagonal ? (int)(((int64_t)q + tx) % a.tiles_r) : q;
    r0 = ty * TILE;
    c0 = tx * TILE;
}

__device__ __forceinline__ bool whole_tile(const MoveArgs &a, int r0, int c0) {
    return r0 + TILE <= a.rows && c0 + TILE <= a.cols;
}

// ---------------------------------------------------------------- copy

__global__ void __launch_bounds__(THREADS) k_copy(MoveArgs a) {
    int r0, c0;
    tile_origin(a, r0, c0);
    const uint32_t *__restrict__ in = a.in;  // the host rejects overlapping buffers
    uint32_t *__restrict__ out = a.out;
    const int tid = threadIdx.x;
    if (a.vec_ok && whole_tile(a, r0, c0)) {
        const int q = tid % CHUNKS_PER_ROW, r = tid / CHUNKS_PER_ROW;
        u32x4 v[TILE / VEC_ROWS_PER_PASS];
#pragma unroll
        for (int i = 0; i < TILE / VEC_ROWS_PER_PASS; i++)
            v[i] = __builtin_nontemporal_load(
                (const u32x4 *)(in + (int64_t)(r0 + r + i * VEC_ROWS_PER_PASS) * a.ldi + c0 + 4 * q));
#pragma unroll
        for (int i = 0; i < TILE / VEC_ROWS_PER_PASS; i++)
            __builtin_nontemporal_store(
                v[i], (u32x4 *)(out + (int64_t)(r0 + r + i * VEC_ROWS_PER_PASS) * a.ldo + c0 + 4 * q));
        return;
    }
    const int lane = tid & 63, wave = tid >> 6;
    const int c = c0 + lane;
    for (int j = 0; j < TILE; j += ROWS_PER_PASS) {
        const int r = r0 + wave + j;
        if (r < a.rows && c < a.cols) out[(int64_t)r * a.ldo + c] = in[(int64_t)r * a.ldi + c];
    }
}

// ---------------------------------------------------------------- naive

__global__ void __launch_bounds__(THREADS) k_transpose_naive(MoveArgs a) {
    int r0, c0;
    tile_origin(a, r0, c0);
    const uint32_t *__restrict__ in = a.in;  // the host rejects overlapping buffers
    uint32_t *__restrict__ out = a.out;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = c0 + lane;
    if (whole_tile(a, r0, c0)) {
        // all loads of the tile in flight before the first store
        uint32_t v[TILE / ROWS_PER_PASS];
#pragma unroll
        for (int j = 0; j < TILE / ROWS_PER_PASS; j++)
            v[j] = in[(int64_t)(r0 + wave + j * ROWS_PER_PASS) * a.ldi + c];
#pragma unroll
        for (int j = 0; j < TILE / ROWS_PER_PASS; j++)
            out[(int64_t)c * a.ldo + r0 + wave + j * ROWS_PER_PASS] = v[j];
        return;
    }
    for (int j = 0; j < TILE; j += ROWS_PER_PASS) {
        const int r = r0 + wave + j;
        if (r < a.rows && c < a.cols) out[(int64_t)c * a.ldo + r] = in[(int64_t)r * a.ldi + c];
    }
}

// ---------------------------------------------------------------- LDS tile

enum { LAYOUT_PLAIN = 0, LAYOUT_PADDED = 1, LAYOUT_SWIZZLED = 2 };

template <int LAYOUT>
struct TileLayout {
    static constexpr int WORDS = LAYOUT == LAYOUT_PADDED ? TILE * (TILE + 1) : TILE * TILE;
    // Word index of tile element (r, c) (input row r, input column c).
    __device__ static __forceinline__ int at(int r, int c) {
        if (LAYOUT == LAYOUT_PADDED) return r * (TILE + 1) + c;
        if (LAYOUT == LAYOUT_SWIZZLED) return r * TILE + (c ^ r);
        return r * TILE + c;
    }
};

// Element-wise tile transpose: rows of the tile in (coalesced, lane = column),
// barrier, columns of the tile out (coalesced, lane = input row).
template <int LAYOUT>
__device__ __forceinline__ void tile_transpose(const MoveArgs &a, int r0, int c0, uint32_t *tile) {
    typedef TileLayout<LAYOUT> L;
    const uint32_t *__restrict__ in = a.in;  // the host rejects overlapping buffers
    uint32_t *__restrict__ out = a.out;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (whole_tile(a, r0, c0)) {
        // all loads of the tile in flight before the first LDS write
        uint32_t v[TILE / ROWS_PER_PASS];
#pragma unroll
        for (int j = 0; j < TILE / ROWS_PER_PASS; j++)
            v[j] = in[(int64_t)(r0 + wave + j * ROWS_PER_PASS) * a.ldi + c0 + lane];
#pragma unroll
        for (int j = 0; j < TILE / ROWS_PER_PASS; j++) tile[L::at(wave + j * ROWS_PER_PASS, lane)] = v[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < TILE / ROWS_PER_PASS; j++) {
            const int oc = wave + j * ROWS_PER_PASS;  // output row within the tile = input column
            out[(int64_t)(c0 + oc) * a.ldo + r0 + lane] = tile[L::at(lane, oc)];
        }
        return;
    }
    for (int j = 0; j < TILE; j += ROWS_PER_PASS) {
        const int r = wave + j;
        if (r0 + r < a.rows && c0 + lane < a.cols)
            tile[L::at(r, lane)] = in[(int64_t)(r0 + r) * a.ldi + c0 + lane];
    }
    __syncthreads();
    for (int j = 0; j < TILE; j += ROWS_PER_PASS) {
        const int oc = wave + j;  // output row within the tile = input column
        if (c0 + oc < a.cols && r0 + lane < a.rows)
            out[(int64_t)(c0 + oc) * a.ldo + r0 + lane] = tile[L::at(lane, oc)];
    }
}

template <int LAYOUT>
__global__ void __launch_bounds__(THREADS) k_transpose_lds(MoveArgs a) {
    __shared__ uint32_t tile[TileLayout<LAYOUT>::WORDS];
    int r0, c0;
    tile_origin(a, r0, c0);
    tile_transpose<LAYOUT>(a, r0, c0, tile);
}

// ---------------------------------------------------------------- vector

// The tile is stored transposed: word (x, y) = input element (row y, column
// x), at x * 64 + (y ^ (x & 60)).  The XOR term is a multiple of 4, so each
// group of four consecutive y stays one aligned 16-byte chunk, and the 16
// lanes that read one x back get 16 distinct chunks: the 16-byte reads are
// conflict-free (measured).  Each wave-wide scalar store touches 16 rows x
// at 64 distinct banks; gfx950 still charges such a store about two
// conflict cycles (measured: its 4-byte stores run conflict-free when each
// 16-lane group writes one contiguous 64-byte run, not when a group's words
// are spread over a row and the rows change between groups).  The store
// side costs no bandwidth here: the transpose is HBM-bound.
__device__ __forceinline__ int vec_at(int x, int y) { return x * TILE + (y ^ (x & 60)); }

__global__ void __launch_bounds__(THREADS) k_transpose_vec(MoveArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t tile[TILE * TILE];
    int r0, c0;
    tile_origin(a, r0, c0);
    if (!(a.vec_ok && whole_tile(a, r0, c0))) {
        tile_transpose<LAYOUT_SWIZZLED>(a, r0, c0, tile);
        return;
    }
    const uint32_t *__restrict__ in = a.in;  // the host rejects overlapping buffers
    uint32_t *__restrict__ out = a.out;
    const int tid = threadIdx.x;
    const int q = tid % CHUNKS_PER_ROW, rr = tid / CHUNKS_PER_ROW;
    u32x4 v[TILE / VEC_ROWS_PER_PASS];
#pragma unroll
    for (int i = 0; i < TILE / VEC_ROWS_PER_PASS; i++)
        v[i] = *(const u32x4 *)(in + (int64_t)(r0 + rr + i * VEC_ROWS_PER_PASS) * a.ldi + c0 + 4 * q);
#pragma unroll
    for (int i = 0; i < TILE / VEC_ROWS_PER_PASS; i++) {
        const int y = rr + i * VEC_ROWS_PER_PASS;  // input row within the tile
#pragma unroll
        for (int e = 0; e < 4; e++) tile[vec_at(4 * q + e, y)] = v[i][e];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TILE / VEC_ROWS_PER_PASS; i++) {
        const int x = rr + i * VEC_ROWS_PER_PASS;  // output row within the tile = input column
        const u32x4 w = *(const u32x4 *)(tile + vec_at(x, 4 * q));
        *(u32x4 *)(out + (int64_t)(c0 + x) * a.ldo + r0 + 4 * q) = w;
    }
}

// ---------------------------------------------------------------- host side

bool overlap(const void *a, uint64_t alen, const void *b, uint64_t blen) {
    if (!alen || !blen) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + blen && y < x + alen;
}

uint64_t span(int64_t rows, int64_t cols, int64_t ld) {
    if (rows == 0 || cols == 0) return 0;
    return (uint64_t)((rows - 1) * ld + cols) * 4u;
}

int launch_move(int method, bool transpose, int64_t rows, int64_t cols, const float *in,
                int64_t ldi, float *out, int64_t ldo, void *stream) {
    if (rows < 0 || cols < 0 || rows > INT32_MAX - TILE || cols > INT32_MAX - TILE)
        return TDG_ERR_INVALID_ARG;
    const int64_t out_cols = transpose ? rows : cols;
    const int64_t out_rows = transpose ? cols : rows;
    if (ldi < (cols > 1 ? cols : 1) || ldo < (out_cols > 1 ? out_cols : 1)) return TDG_ERR_INVALID_ARG;
    // rows x leading dimension must fit in int64 bytes before span() uses it
    if ((rows > 0 && ldi > INT64_MAX / 4 / rows) || (out_rows > 0 && ldo > INT64_MAX / 4 / out_rows))
        return TDG_ERR_INVALID_ARG;
    if (rows > 0 && cols > 0 && (!in || !out)) return TDG_ERR_INVALID_ARG;
    if (overlap(in, span(rows, cols, ldi), out, span(out_rows, out_cols, ldo)))
        return TDG_ERR_INVALID_ARG;
    if (method < TDG_TRANSPOSE_AUTO || method > TDG_TRANSPOSE_VEC) return TDG_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return TDG_OK;
    const int dev = tdg::device_check();
    if (dev != TDG_OK) return dev;

    MoveArgs a;
    a.in = (const uint32_t *)in;
    a.out = (uint32_t *)out;
    a.ldi = ldi;
    a.ldo = ldo;
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.tiles_c = (int)((cols + TILE - 1) / TILE);
    a.tiles_r = (int)((rows + TILE - 1) / TILE);
    a.diagonal = transpose ? 1 : 0;
    const int64_t tiles = (int64_t)a.tiles_r * a.tiles_c;
    if (tiles > INT32_MAX) return TDG_ERR_UNSUPPORTED;
    a.vec_ok = ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0) && ldi % 4 == 0 && ldo % 4 == 0;

    const void *fn;
    if (!transpose) fn = (const void *)&k_copy;
    else if (method == TDG_TRANSPOSE_NAIVE) fn = (const void *)&k_transpose_naive;
    else if (method == TDG_TRANSPOSE_LDS) fn = (const void *)&k_transpose_lds<LAYOUT_PLAIN>;
    else if (method == TDG_TRANSPOSE_LDS_PADDED) fn = (const void *)&k_transpose_lds<LAYOUT_PADDED>;
    else if (method == TDG_TRANSPOSE_LDS_SWIZZLED) fn = (const void *)&k_transpose_lds<LAYOUT_SWIZZLED>;
    else fn = (const void *)&k_transpose_vec;

    void *kargs[] = {&a};
    if (hipLaunchKernel(fn, dim3((unsigned)tiles), dim3(THREADS), kargs, 0, (hipStream_t)stream) !=
        hipSuccess)
        return TDG_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return TDG_ERR_LAUNCH;
    return TDG_OK;
}

}  // namespace

extern "C" {

int tdg_copy_f32(int64_t rows, int64_t cols, const float *in, int64_t ldi, float *out, int64_t ldo,
                 void *stream) {
    return launch_move(TDG_TRANSPOSE_AUTO, false, rows, cols, in, ldi, out, ldo, stream);
}

int tdg_transpose_f32(int method, int64_t rows, int64_t cols, const float *in, int64_t ldi,
                      float *out, int64_t ldo, void *stream) {
    return launch_move(method, true, rows, cols, in, ldi, out, ldo, stream);
}

}  // extern "C"
