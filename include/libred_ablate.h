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
 * an LDS tree as on the page (elements past n count as 0), and then *out =
 * the float64 sum of the partials, rounded once to float32 (the page does
 * this last step on the host). partials_cap is the capacity of `partials` in
 * elements; a capacity below np, a rung outside 1..6, n == 0 or
 * n > 2^31 for rungs 1-5 is RED_ERR_INVALID_ARG.
 */
red_status red_ablate_sum_f32(int rung, const float *x, size_t n, float *partials,
                              size_t partials_cap, float *out, hipStream_t stream);

/* Number of partials rung 1-5 writes for n elements (0 for another rung). */
size_t red_ablate_num_partials(int rung, size_t n);

/*
 * Launch shape of the single-value kernels: `block` threads per block (256,
 * 512 or 1024), at most `blocks_per_cu` blocks per compute unit, `unroll`
 * independent 16-byte loads per thread per loop trip (1, 2, 4, 8 or 16),
 * `nontemporal` 1 to mark the streaming loads non-temporal.
 */
typedef struct red_flat_policy {
    int block;
    int blocks_per_cu;
    int unroll;
    int nontemporal;
} red_flat_policy;

/* Launch shape of the row kernels: `block` threads (64, 128, 256 or 512; one
 * row per wave at a time), `unroll` loads per lane per trip (1, 2, 4 or 8),
 * `nontemporal`, and `max_blocks` capping the grid. */
typedef struct red_rows_policy {
    int block;
    int unroll;
    int nontemporal;
    int max_blocks;
} red_rows_policy;

/* The shapes red_sum_f32 / red_sum_i32_i64 / red_max_f32 and the row entry
 * points use. */
void red_default_flat_policy(red_flat_policy *p);
void red_default_rows_policy(red_rows_policy *p);

/* The number of blocks a single-value call of n elements launches with
 * policy p (NULL = default) on the current device; 0 on error. */
size_t red_flat_grid(size_t n, const red_flat_policy *p);

/* The single-value and row entry points with an explicit launch shape.
 * An unsupported shape is RED_ERR_INVALID_ARG. Results obey the same
 * contracts as the default entry points. */
red_status red_sum_f32_with(const float *x, size_t n, float *out, const red_flat_policy *p,
                            hipStream_t stream);
red_status red_sum_i32_i64_with(const int32_t *x, size_t n, int64_t *out,
                                const red_flat_policy *p, hipStream_t stream);
red_status red_max_f32_with(const float *x, size_t n, float *out, const red_flat_policy *p,
                            hipStream_t stream);
red_status red_rows_sum_f32_with(const float *x, size_t rows, size_t cols, float *out,
                                 const red_rows_policy *p, hipStream_t stream);
red_status red_rows_max_f32_with(const float *x, size_t rows, size_t cols, float *out,
                                 const red_rows_policy *p, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBRED_ABLATE_H_ */
