/*
 * libred_ablate.h -- the ablation ladder and explicit launch shapes.
 *
 * These entry points exist to measure the design, not for production use.
 * Their conventions are those of libred.h (device pointers, asynchronous on
 * `stream`, argument errors returned before any HIP call).
 */
#ifndef LIBRED_ABLATE_H_
#define LIBRED_ABLATE_H_

#include "libred.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The five block-reduction versions of the reduction lesson
 * ("03_shared_memory_sync_reduction.py -- shared memory, banks,
 * synchronisation and parallel reduction", demo 3), on 256-thread blocks:
 *   1 interleaved addressing with divergent branches,
 *   2 interleaved addressing by consecutive threads (LDS bank conflicts),
 *   3 sequential addressing,
 *   4 first add during the load (each block covers 512 elements),
 *   5 version 4 finished by one 64-lane wave with register shuffles.
 * Rung 6 is the production path of red_sum_f32 (partials unused).
 *
 * Rungs 1-5 write one float32 partial per block into partials[0..np), where
 * np = red_ablate_num_partials(rung, n), each partial summed in float32 by
 * an LDS tree as on the page (elements past n count as 0). Then, unless out
 * is NULL, *out = the float64 sum of the partials rounded once to float32
 * (the page does this last step on the host; here red_sum_f32 does it on
 * the device). With out == NULL only the rung's own kernel runs, which is
 * how it is timed. partials_cap is the capacity of `partials` in elements;
 * a capacity below np, a rung outside 1..6, n == 0, n > 2^31 for rungs 1-5,
 * or a NULL out for rung 6 is RED_ERR_INVALID_ARG.
 */
red_status red_ablate_sum_f32(int rung, const float *x, size_t n, float *partials,
                              size_t partials_cap, float *out, hipStream_t stream);

/* Number of partials rung 1-5 writes for n elements (0 for another rung). */
size_t red_ablate_num_partials(int rung, size_t n);

/*
 * Launch shape of the single-value kernels.
 *   block          threads per block
 *   blocks_per_cu  at most this many blocks per compute unit
 *   unroll         independent 16-byte loads per lane per loop trip
 *   nontemporal    1: mark the streaming loads non-temporal
 *   layout         0: grid-stride (thread i reads vectors i, i + G*T, ...);
 *                  1: wave tiles (each wave reads whole tiles of 64*unroll
 *                     contiguous vectors, tiles dealt round-robin to waves)
 *   prefetch       layout 1 only: issue the next tile's loads before folding
 *                  the current tile
 *   combine        0: the last block to finish combines the partials in the
 *                  same launch; 1: a second one-block launch combines them
 * Compiled shapes: layout 0 with block 256/1024 and unroll 1/4/8
 * (prefetch 0); layout 1 with block 64/256/1024 and unroll 4/8/16 (every
 * default shape, and a small set around them). Others are
 * RED_ERR_INVALID_ARG.
 */
typedef struct red_flat_policy {
    int block;
    int blocks_per_cu;
    int unroll;
    int nontemporal;
    int layout;
    int prefetch;
    int combine;
} red_flat_policy;

/* Launch shape of the row kernels: `block` threads (64, 128, 256 or 512; one
 * row per wave at a time), `unroll` loads per lane per trip (1, 2, 4, 8, 16),
 * `nontemporal`, `max_blocks` capping the grid (the one-wave-per-row grid is
 * then trimmed so that every wave gets the same number of rows, give or take
 * one), `split`: 0 = split few long rows across single-wave blocks when that
 * helps (the default rule), 1 = never, 2 = whenever a row holds at least two
 * tiles of 64*unroll vectors; `cover` (one wave per row): 0 = rows that do
 * not all start 16-byte aligned are read as the aligned 16-byte vectors
 * that cover each row, with every load unconditional and the elements
 * outside the row masked when folded (rows of at least 16 elements), and
 * aligned rows directly; 1 = never (each row peels its unaligned head and
 * tail element by element); 2 = always; `prefetch` (0 or 1, one wave per
 * row, rows of at least 16 elements): a single-wave streaming kernel that
 * reads rows through their covers and keeps the next tile of 64*unroll
 * vectors in flight while folding the current one, across row boundaries;
 * and `short_rows`, the kernels for short rows (`block` and `prefetch` do
 * not apply to them, `max_blocks` caps their grid, an `unroll` of 8 or 16
 * gives the LDS-staged kernel tiles of that many 16-byte vectors per lane
 * when that is more than the rows need, and the LDS-staged kernel always
 * loads non-temporally, whatever `nontemporal` says):
 *   0  the library's choice: rows of 1 to 32 floats of a contiguous,
 *      16-byte aligned matrix go to the narrow kernel (17); other rows of
 *      fewer than 1024 floats go to the
 *      LDS-staged kernel when they are contiguous or their gaps (ld - cols)
 *      hold at most a quarter of a row (or, for rows of 3 to 128 floats,
 *      at most 64 floats), and the matrix spans at least 8
 *      elements (any alignment of x: the first and last vectors of the
 *      matrix are read element by element when they reach outside it); it
 *      loads tiles of rows, gaps included, as 16-byte vectors whatever the
 *      row length and then reduces each row from LDS with a power of two of
 *      lanes; other rows of at most 512 floats go to the packed kernel, which gives
 *      each row a segment of up to 16 lanes (16-byte units, rows 16-byte
 *      aligned) or 64 lanes (single elements), so that one load covers
 *      several rows;
 *   1  neither;
 *   2  the packed kernel only (rows of at most 512 floats);
 *   3-9  the LDS-staged kernel with 2^(short_rows - 3) lanes per row where it
 *      applies (as for 0, at any row length whose tile fits 4096 floats:
 *      for a contiguous, 16-byte aligned matrix, 4 rows of an odd width, 2
 *      of a width of 2 mod 4, or 1 row; otherwise one row plus 3), else as
 *      2;
 *   10-16  the same with 2^(short_rows - 10) lanes per row, which read
 *      16-byte vectors from LDS when the rows hold whole vectors that start
 *      16-byte aligned (cols and ld multiples of 4, x 16-byte aligned; the
 *      default for such rows of at most 64 floats);
 *   17  the narrow kernel for rows of 1 to 32 floats of a contiguous,
 *      16-byte aligned matrix (each lane folds the whole rows of its own
 *      16-byte vectors, read through LDS when they span several; tiles of
 *      at least 8 coalesced loads per lane; the library's choice), else as
 *      0;
 * and `defer`: for the LDS-staged kernel, 0 or 2 = a wave keeps its row
 * results in LDS and stores them after its last tile when they fit beside
 * its staging tile in its share of the CU's LDS (the CU's LDS over the waves
 * the grid puts on each CU, and at most one block's limit), else stores
 * each tile's results as the tile is reduced; 1 = always as each tile is
 * reduced; for the narrow kernel, 0 = a wave holds the results of several
 * tiles (up to 48 KiB) in LDS and stores them in one burst, for rows of 6
 * and of 8 to 32 floats, and stores each tile's results as the tile is
 * reduced otherwise; 1 = always as each tile is reduced; 2 = always held. The
 * results are the same either way; and `lines` (the LDS-staged kernel, a
 * contiguous, 16-byte aligned matrix): 0 = the library's choice (1 for rows
 * of fewer than 32 floats), 1 = tiles of a multiple of 32 rows (whole
 * 128-byte lines of input and of output when x and out are 128-byte
 * aligned), 2 = as many rows as fit; and `xcd`, which blocks of the
 * one-wave-per-row, streaming, packed and LDS-staged kernels run on which
 * of the 8 XCDs (the launch deals block b to XCD b mod 8): 1 = block b takes
 * the rows (or tiles) of index b; n = 2-4096: the indices are dealt to the
 * XCDs in runs of n consecutive ones, the grid rounded up to a multiple of
 * 8n when it has at least 8n blocks (else as 1), so that a row and the next,
 * which share the 128-byte line where one ends, are mostly read on one XCD;
 * 0 = the library's choice (runs of 64 for rows of 768 to 4095 floats that
 * do not all start on a 128-byte line, else 1). The results are the same
 * either way; and `max_fold`, how the LDS-staged kernel's maxima fold a
 * lane's elements: 1 = a compare and a select, 2 = a hardware max of the
 * canonicalized element (a signalling NaN is made quiet first, so a NaN
 * never wins either way) with up to 4 lanes per row, and the compare and
 * select with more, 0 = the library's choice (2 for rows of fewer than 64
 * floats, else 1). The results are the same either way. */
typedef struct red_rows_policy {
    int block;
    int unroll;
    int nontemporal;
    int max_blocks;
    int split;
    int prefetch;
    int short_rows;
    int cover;
    int defer;
    int lines;
    int xcd;
    int max_fold;
} red_rows_policy;

/* Launch shape of the column kernels: `unroll` rows in flight per lane (1, 2,
 * 4, 8 or 16), `nontemporal` (the shifted vectors described under `vec` are
 * always loaded non-temporally), `target_waves` (the rows are cut into chunks
 * until about this many single-wave blocks run), `vec`: 0 = four adjacent
 * columns per lane: from one aligned 16-byte load per row when x is 16-byte
 * aligned and cols and ld are multiples of 4, or through an m-row view (see
 * `fold`); else, with at least 4 columns, from the aligned vector each
 * lane's first column lies in and the next one, which the lane takes from
 * the lane that loaded it (lane l + 1), so that each block's last group of
 * four columns, or a packed row's, only lends its vector (no lane reads
 * past the vector that holds its row's last column); under 4 columns of
 * such rows, one column per lane; 1 = always one; 4 = same as 0; `fold`
 * (with vec 0 or 4, for a contiguous
 * (ld == cols) matrix): the matrix is read as view rows of m * cols columns,
 * m consecutive rows as one, with four columns per lane, starting at x or,
 * when x is not 16-byte aligned, at the next 128-byte boundary (so that such
 * a matrix is read four columns per lane too, even with m = 1), and a
 * second pass adds each column's m partial columns and then its elements
 * after the last whole view row and before the view. m must make every m-row span start 16-byte aligned (a
 * multiple of 4 / gcd(cols, 4)). 0 = the library's choice (for widths of
 * at least 256 that are not a multiple of 32, with at least 32768 rows: 32,
 * so that each view row spans whole 128-byte lines, except for widths of
 * 2 mod 4, which take 16; 16 for the other widths of at least 256 that are
 * not a multiple of 4; for widths of 32 to 255, the smallest m that is a
 * multiple of 32 / gcd(cols, 32) and whose view rows hold 512 groups of
 * four columns, at most 64, unless the width is a multiple of 4 whose own
 * rows keep 95% of the lanes busy; below 32 columns, the smallest multiple
 * of 32 / gcd(cols, 32) up to 32 (16 for multiples of 4) that keeps 84% of
 * the lanes busy, when the choice below keeps fewer than 99%; otherwise the
 * m up to 16 that leaves the fewest lanes idle, multiples of 4 folded only
 * for 5% more lanes), 1 =
 * never, 2-64 = that m, rounded up to a valid multiple and down to the
 * rows; and `width` (1, 2 or 4):
 * with at least 64 column groups, each row is read by `width` loads per lane,
 * so a wave reads width x 1 KiB (four columns per lane) or width x 256 bytes
 * (one column per lane) of a row at once (with fewer groups, 1 is used);
 * `prefetch` (0 or 1): issue the next group of `unroll` rows before adding
 * the current one; `order`, which rows each of the n row phases takes and
 * in what order: 1 = every n-th group of rows, each phase from the top, so
 * a launch reads one band of the matrix at a time; 2 = the same rows, but
 * block b starts at its (b mod m)-th of m groups and wraps around to the
 * first, so the waves read rows spread over the matrix; 3 = one run of
 * consecutive rows per phase (about rows / n); 0 = the library's choice
 * (when the row pitch as read, ld or the view's, is a multiple of 255 or
 * 257 floats, pitches whose band reads fill a few memory channels' queues:
 * 3 for a matrix read unfolded, 2 through an m-row view;
 * 3 when a wave's load covers several rows (fewer than 64 column groups)
 * whose bytes are not a whole number of 128-byte lines, so that the line two
 * loads share is read by one wave; else 1). The order changes the order in which a column's elements are
 * added, never the fact that the result is fixed by the shape. `xcd`: which
 * blocks run on which of the 8 XCDs (the launch deals block b to XCD
 * b mod 8): 1 = block b takes column block b mod n of phase b / n (n column
 * blocks); 2 = the blocks of each XCD take one contiguous range of the
 * indices j + k * n (column block j of phase k), so that the 128-byte line
 * two column blocks, or two adjacent rows, share is fetched into one XCD's
 * L2; 0 = the library's choice: 2 with at least 8 phases, rounded down to a
 * multiple of 8 (each XCD then holds every column block of whole phases)
 * when that keeps three quarters of them, unless the row pitch as read is
 * a power of two bytes; else 1. */
typedef struct red_cols_policy {
    int unroll;
    int nontemporal;
    int target_waves;
    int vec;
    int width;
    int prefetch;
    int fold;
    int order;
    int xcd;
} red_cols_policy;

/* The default column shape. A call without a policy uses it, except on
 * short-wide matrices (four columns per lane and cols / 256 > 1024, cols of
 * the m-row view when folded), and on unfolded matrices of at least 256
 * columns whose rows are not a whole number of 128-byte lines, which use
 * unroll 2, width 4, no prefetch and target_waves 1024 (short-wide ones
 * with their row phases rounded down so that the grid holds at most 1024
 * blocks, and with the prefetch where it then holds at most 640); with one column
 * per lane and at least 64 columns, which use unroll 8, width 2, no
 * prefetch and target_waves 2048; and on rows that do not start 16-byte
 * aligned (four columns per lane from shifted vectors), which use unroll 4,
 * width 2, prefetch and target_waves 1024 with at least 63 groups of four
 * columns, else unroll 8, prefetch and target_waves 2048; and on m-row views
 * (see `fold`) of at most 224 blocks of 256 view columns whose default
 * launch would leave too few row phases for the XCD grouping of `xcd` 0,
 * which use unroll 4, prefetch and target_waves 1024; and on unfolded
 * rows of more than 8192 columns (at most 1024 blocks of 256, a pitch that
 * is not a power of two bytes), which use unroll 4, width 2, no prefetch
 * and target_waves 1024, unless the shape above would have its blocks
 * grouped per XCD and this one would not (with 128 or more blocks per
 * phase, their phases are rounded down where that keeps at least 864
 * blocks, or leaves at most 640, then with the prefetch). */
void red_default_cols_policy(red_cols_policy *p);
red_status red_cols_sum_f32_with(const float *x, size_t rows, size_t cols, size_t ld, float *out,
                                 const red_cols_policy *p, hipStream_t stream);
red_status red_cols_max_f32_with(const float *x, size_t rows, size_t cols, size_t ld, float *out,
                                 const red_cols_policy *p, hipStream_t stream);

/* The shape red_sum_f32 / red_sum_i32_i64 / red_max_f32 use for n elements
 * (up to 2^15 elements, one block of 1024 threads that stores the result
 * itself). */
void red_default_flat_policy(size_t n, red_flat_policy *p);
/* The default shape of the row entry points for aligned rows of 2048 to 16383
 * floats. A call without a policy adapts it to the row length: 16 loads per
 * lane and max_blocks 512 from 16384 floats up; 4 loads per lane and
 * max_blocks 2048 for rows of 2049 to 4095 floats whose last 2048-float tile
 * is at most 75% full; below 2048 floats, at most 4
 * loads per lane (a tile no longer than the row) and max_blocks 2048. Rows
 * read through their covers take 8 loads per lane and max_blocks 32768 below
 * 16384 floats, and 8 and 1024 from there. */
void red_default_rows_policy(red_rows_policy *p);

/* The number of blocks a single-value call of n elements launches with
 * policy p (NULL = default) on the current device; 0 on error. */
size_t red_flat_grid(size_t n, const red_flat_policy *p);

/*
 * Steps 1-5 of red_sum_f32 alone: each block of the launch (policy p, NULL =
 * the default for n) stores its float64 partial; *count receives the number
 * of blocks np = red_flat_grid(n, p), and partials[0..np) the partials in
 * block order. Their sum is the sum of x[0..n). No final combine is run and
 * the library workspace is not used. partials_cap < np, a NULL partials or
 * count, or partials overlapping x is RED_ERR_INVALID_ARG.
 */
red_status red_sum_f32_partials(const float *x, size_t n, double *partials, size_t partials_cap,
                                const red_flat_policy *p, size_t *count, hipStream_t stream);

/* Operation codes for red_flat_with. */
enum {
    RED_OP_SUM_F32 = 0,     /* float in, float out (red_sum_f32) */
    RED_OP_SUM_I32_I64 = 1, /* int32_t in, int64_t out */
    RED_OP_MAX_F32 = 2,     /* float in, float out */
    RED_OP_MIN_F32 = 3,     /* float in, float out */
    RED_OP_ARGMAX_F32 = 4,  /* float in, int64_t out */
    RED_OP_ARGMIN_F32 = 5,  /* float in, int64_t out */
    RED_OP_SUM_BF16_F32 = 6,/* uint16_t (bfloat16 bits) in, float out */
    RED_OP_SUM_F16_F32 = 7, /* uint16_t (IEEE half bits) in, float out */
    RED_OP_SUM_F64 = 8,     /* double in, double out */
    RED_OP_SUM_MAX_F32 = 9  /* float in, float[3] out (red_sum_max_f32) */
};

/* Any single-value operation with an explicit launch shape: x and out have
 * the element types listed for `op`; contracts as for the plain entry
 * point. An unknown op or an unsupported shape is RED_ERR_INVALID_ARG. */
red_status red_flat_with(int op, const void *x, size_t n, void *out, const red_flat_policy *p,
                         hipStream_t stream);

/* The single-value and row entry points with an explicit launch shape.
 * An unsupported shape is RED_ERR_INVALID_ARG. Results obey the same
 * contracts as the default entry points. */
red_status red_sum_f32_with(const float *x, size_t n, float *out, const red_flat_policy *p,
                            hipStream_t stream);
red_status red_sum_i32_i64_with(const int32_t *x, size_t n, int64_t *out,
                                const red_flat_policy *p, hipStream_t stream);
red_status red_max_f32_with(const float *x, size_t n, float *out, const red_flat_policy *p,
                            hipStream_t stream);
red_status red_sum_max_f32_with(const float *x, size_t n, float *out3, const red_flat_policy *p,
                                hipStream_t stream);
red_status red_rows_sum_f32_with(const float *x, size_t rows, size_t cols, size_t ld, float *out,
                                 const red_rows_policy *p, hipStream_t stream);
red_status red_rows_max_f32_with(const float *x, size_t rows, size_t cols, size_t ld, float *out,
                                 const red_rows_policy *p, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBRED_ABLATE_H_ */
