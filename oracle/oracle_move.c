/*
 * oracle_move.c -- the plain CPU oracle for the copy / transpose ladder.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU product
 * path never links, loads or calls it; the two share no code.
 *
 * What it computes ("fixing GPU kernels by hand", the four-step transpose
 * exercise): for a rows x cols matrix `in` (row-major, leading dimension
 * ldi),
 *   copy:       out[i][j] = in[i][j]      (out rows x cols, leading dim ldo)
 *   transpose:  out[j][i] = in[i][j]      (out cols x rows, leading dim ldo)
 * Elements are moved as 32-bit patterns: no arithmetic touches them, so NaN
 * payloads, signed zeros and subnormals come out exactly as they went in.
 * The loops run in plain row order; nothing is blocked or reordered.
 *
 * Return value: 0 on success, -1 on invalid arguments.
 */
#include <stddef.h>
#include <stdint.h>

static int check(int64_t rows, int64_t cols, const void *in, int64_t ldi, const void *out,
                 int64_t ldo, int64_t out_cols)
{
    if (rows < 0 || cols < 0) return -1;
    if (ldi < (cols > 1 ? cols : 1) || ldo < (out_cols > 1 ? out_cols : 1)) return -1;
    if (rows > 0 && cols > 0 && (!in || !out)) return -1;
    return 0;
}

int oracle_copy_u32(int64_t rows, int64_t cols, const uint32_t *in, int64_t ldi, uint32_t *out,
                    int64_t ldo)
{
    if (check(rows, cols, in, ldi, out, ldo, cols)) return -1;
    for (int64_t i = 0; i < rows; i++)
        for (int64_t j = 0; j < cols; j++)
            out[i * ldo + j] = in[i * ldi + j];
    return 0;
}

int oracle_transpose_u32(int64_t rows, int64_t cols, const uint32_t *in, int64_t ldi,
                         uint32_t *out, int64_t ldo)
{
    if (check(rows, cols, in, ldi, out, ldo, rows)) return -1;
    for (int64_t i = 0; i < rows; i++)
        for (int64_t j = 0; j < cols; j++)
            out[j * ldo + i] = in[i * ldi + j];
    return 0;
}
