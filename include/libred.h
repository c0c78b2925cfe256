/*
 * libred.h -- block-level parallel reductions for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the reduction lesson develops step by step
 * ("03_shared_memory_sync_reduction.py -- shared memory, banks,
 * synchronisation and parallel reduction", demo 3): reduce n values to one,
 * with each thread block producing a partial and the partials then combined.
 * Here the whole reduction, including the combine, runs on the GPU.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All data pointers are DEVICE pointers (memory of the current HIP device,
 *    e.g. from hipMalloc or a PyTorch CUDA tensor). The caller allocates and
 *    frees them; the library never frees caller memory.
 *  - Inputs are contiguous, element-aligned arrays (4-byte aligned for float
 *    and int32; 8-byte aligned for the int64 output). Any such address is
 *    accepted: the 16-byte vector body is peeled internally.
 *  - Lengths are size_t; at most RED_MAX_N elements per call.
 *  - Calls are asynchronous: work is enqueued on `stream` (0 = the null
 *    stream) and the call returns without waiting. The result is valid once
 *    the stream has reached that point. A fault in a kernel surfaces at the
 *    caller's next synchronisation.
 *  - Argument errors are reported as RED_ERR_INVALID_ARG before any HIP call
 *    is made: a null input with a non-zero length, a null output, a
 *    misaligned pointer, an output that overlaps the input, a length above
 *    RED_MAX_N, or rows * cols overflowing. Nothing is enqueued then.
 *  - The single-value entry points use a small workspace owned by the library
 *    (block partials plus a completion counter), allocated on the first call
 *    per (device, stream) and kept until the process exits. Calls on one
 *    stream are ordered, so they can share it; eager calls on different
 *    streams use different workspaces and may run concurrently. The column
 *    entry points keep their partials in a per-stream scratch buffer under
 *    the same rule. The library allocates with the calling thread in relaxed
 *    capture mode, so a first call on a stream that is not being captured
 *    does not disturb a capture under way on another stream.
 *  - Graph capture: the calls can be captured into a HIP graph, provided the
 *    stream already holds what the call needs. That is its workspace, made by
 *    any earlier single-value call on the stream (row calls need it only
 *    when they split long rows). For the column entry points it is also
 *    scratch at least as large as the call needs, made by an earlier column
 *    call of the same or a larger shape. Otherwise the
 *    call returns RED_ERR_CAPTURE before it touches the stream, and the
 *    capture stays intact. Workspace and scratch are never freed while the
 *    process runs (outgrown scratch included), so a captured graph stays
 *    valid after later calls on its stream.
 *  - A captured graph keeps the workspace and scratch of its capture stream.
 *    It must therefore not run at the same time as other work on that
 *    stream's buffers: eager calls still enqueued on the capture stream, or
 *    another graph captured on the same stream with the same buffers. To
 *    replay graphs concurrently, give each capture buffers of its own with
 *    red_stream_new_workspace between the captures.
 *  - Results are deterministic: for a given length and device the partials
 *    are combined in a fixed index order, so repeated calls return the same
 *    bits.
 *  - Nothing throws across this interface.
 */
#ifndef LIBRED_H_
#define LIBRED_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum red_status {
    RED_OK = 0,
    RED_ERR_INVALID_ARG = 1, /* bad pointer, length, shape or alignment */
    RED_ERR_NO_DEVICE = 2,   /* no usable HIP device is current */
    RED_ERR_HIP = 3,         /* a HIP call or kernel launch failed; see red_last_hip_error */
    RED_ERR_ALLOC = 4,       /* the library workspace could not be allocated */
    RED_ERR_CAPTURE = 5,     /* the stream is being captured into a graph and the call
                                would first have to allocate its workspace or scratch */
    RED_ERR_SCRATCH = 6      /* red_sum_f32_noalloc: the launch needs more block partials
                                than its fixed device array holds */
} red_status;

/* Largest element count accepted by one call (2^40 elements, 4 TiB of float). */
#define RED_MAX_N ((size_t)1 << 40)

/*
 * Sum of n float32 values: *out = x[0] + ... + x[n-1], rounded once to float.
 *
 * The reduction lesson's demo 3 computes this sum with block partials and
 * checks it against the float64 sum of the same inputs. Here every element
 * is widened to float64 as it is loaded and all partials stay in float64, so
 * the only float32 rounding is the final one; the result is within about one
 * float32 rounding of the exact sum (far inside |error| <= 1e-5 * sum|x|).
 * NaN or infinite inputs follow IEEE arithmetic. n == 0 stores 0.0f (x may
 * then be NULL).
 */
red_status red_sum_f32(const float *x, size_t n, float *out, hipStream_t stream);

/*
 * red_sum_f32 for callers that cannot allocate device memory: code being
 * captured into a HIP graph on a stream that holds no workspace yet, serving
 * loops that must not allocate, harnesses that forbid hipMalloc. Same
 * arguments, kernels, launch shapes and result bits as red_sum_f32 (n, x,
 * out, stream; errors as there). It calls no hipMalloc, hipFree or other
 * allocating routine: the block partials go to a fixed array of 4096
 * float64 values (32 KiB) in device memory, one per device, held until the
 * process exits. A launch that would need more partials than that returns
 * RED_ERR_SCRATCH before anything is enqueued (on MI355X the default shapes
 * launch at most 2 blocks per compute unit, 512 in all). Every call on one
 * device shares that device's array, and each call overwrites the partials
 * it reads before reading them, so nothing in it needs clearing; but calls
 * that overlap in time on one device (on different streams, or graphs
 * replayed concurrently) race on it and may return wrong sums: order them.
 */
red_status red_sum_f32_noalloc(const float *x, size_t n, float *out, hipStream_t stream);

/*
 * Sum of n int32 values into one int64: *out = x[0] + ... + x[n-1], exact
 * (each element is sign-extended to 64 bits before it is added). This is the
 * reduction of the lesson's demo 3 (block partials, then their sum) over
 * integers: the lesson's own inputs are small integers (i mod 7), summed
 * exactly. Integer addition is associative, so the result is the same
 * whatever the block order, which the simulator page "simt_lab.py" (section
 * 5, launch) asks of every kernel; its shared memory holds only 4-byte words,
 * so the 64-bit accumulator is this library's choice (exact for every int32
 * input). The sum wraps modulo 2^64 only if it leaves the int64 range, which
 * needs n > 2^32. n == 0 stores 0.
 */
red_status red_sum_i32_i64(const int32_t *x, size_t n, int64_t *out, hipStream_t stream);

/*
 * Maximum of n float32 values. The running maximum is replaced only by a
 * strictly greater value (the rule of the SIMT simulator page "simt.py",
 * section 2, DeviceArray.atomic_max), starting from -inf: a NaN never
 * wins, and an empty or all-NaN input gives -inf. Between -0 and +0 either
 * may be returned; they compare equal.
 */
red_status red_max_f32(const float *x, size_t n, float *out, hipStream_t stream);

/*
 * Minimum of n float32 values: the mirror of red_max_f32 (replaced only by a
 * strictly smaller value, from +inf; a NaN never wins; empty or all-NaN gives
 * +inf).
 */
red_status red_min_f32(const float *x, size_t n, float *out, hipStream_t stream);

/*
 * Index of the maximum / minimum of n float32 values: *out = the lowest index
 * i such that x[i] is not NaN and x[i] >= (resp. <=) every non-NaN element;
 * -1 when no element is a number (n == 0 included). Ties go to the lowest
 * index and -0 equals +0, so the answer is unique and independent of the
 * order in which blocks finish. The candidate (value, index) pairs are
 * combined on the device like the partials of red_max_f32.
 */
red_status red_argmax_f32(const float *x, size_t n, int64_t *out, hipStream_t stream);
red_status red_argmin_f32(const float *x, size_t n, int64_t *out, hipStream_t stream);

/*
 * Sum of n 16-bit floats given as their bit patterns (2-byte aligned), into
 * one float32. Each element is widened exactly (bfloat16: the upper half of a
 * float32; IEEE half: the binary16 value); eight elements arrive per 16-byte
 * load. The eight values of a load are first added in float32 as a balanced
 * tree (at most three roundings on any path, each within 2^-24 of the
 * magnitudes added), and each load's total then enters float64 accumulators.
 * bfloat16 values (float32's range) are scaled by 1/8 before the tree, which
 * is exact for every bfloat16 and keeps eight values from overflowing, and
 * the total is scaled back by 8 in float64; eight IEEE halves cannot
 * overflow. Both round once to float32 at the end, far inside
 * |error| <= 1e-5 * sum|x|. NaN/inf and n == 0 as for red_sum_f32.
 */
red_status red_sum_bf16_f32(const uint16_t *x, size_t n, float *out, hipStream_t stream);
red_status red_sum_f16_f32(const uint16_t *x, size_t n, float *out, hipStream_t stream);

/*
 * Sum of n float64 values (8-byte aligned), accumulated in float64 in a fixed
 * order: the error is at most of the order of h * 2^-53 * sum|x_i| with h the
 * longest chain of additions (a few hundred at most), and repeated calls
 * return the same bits.
 */
red_status red_sum_f64(const double *x, size_t n, double *out, hipStream_t stream);

/*
 * Sum, max and sum of magnitudes of n float32 values in one pass over x:
 * out3[0] = x[0] + ... + x[n-1] (as red_sum_f32), out3[1] = the maximum (as
 * red_max_f32), out3[2] = |x[0]| + ... + |x[n-1]| (float64 inside, rounded
 * once; NaN if any x is NaN, +inf if any is infinite). One read of the data
 * yields all three, so sum and max together cost what one of them costs.
 * out3 must hold 3 floats and must not overlap x. n == 0 stores 0, -inf, 0.
 * This fuses the lesson's reduction with the simulator page's max rule; the
 * sum of magnitudes is the scale against which a float sum's error is judged.
 * Its default launch shape differs from red_sum_f32's on large arrays (more
 * waves per CU for the extra arithmetic).
 */
red_status red_sum_max_f32(const float *x, size_t n, float *out3, hipStream_t stream);

/*
 * Per-row sum of a rows x cols float32 matrix stored row-major and
 * contiguously (row r is x[r*cols .. r*cols + cols)):
 * out[r] = x[r*cols] + ... + x[r*cols + cols - 1], for r < rows.
 * One output per segment, as the lesson's block partials are one output
 * per block. Accumulated in float64, rounded once per row. rows == 0 does
 * nothing (out may be NULL); cols == 0 stores 0.0f in every out[r].
 */
red_status red_rows_sum_f32(const float *x, size_t rows, size_t cols, float *out,
                            hipStream_t stream);

/*
 * Per-row maximum of the same layout, with the rule of red_max_f32 applied
 * to each row; cols == 0 stores -inf in every out[r].
 */
red_status red_rows_max_f32(const float *x, size_t rows, size_t cols, float *out,
                            hipStream_t stream);

/*
 * The same row reductions over rows that start `ld` elements apart
 * (ld >= cols): row r is x[r*ld .. r*ld + cols). The elements between the
 * end of one row and the start of the next never enter a result (rows that
 * do not start 16-byte aligned are read as the aligned 16-byte vectors that
 * cover them, which may load up to 3 of those elements on either side of a
 * row, always inside the span x[0 .. (rows - 1) * ld + cols); nothing
 * outside the span is read). ld < cols, or a
 * span (rows - 1) * ld + cols above RED_MAX_N, is RED_ERR_INVALID_ARG. With
 * ld == cols these are red_rows_sum_f32 / red_rows_max_f32. For fewer than
 * 1024 rows of at least 8192 elements, each row is split across several
 * blocks and the pieces are combined per row in a fixed order (this uses the
 * library workspace of the stream).
 */
red_status red_rows_sum_f32_ld(const float *x, size_t rows, size_t cols, size_t ld, float *out,
                               hipStream_t stream);
red_status red_rows_max_f32_ld(const float *x, size_t rows, size_t cols, size_t ld, float *out,
                               hipStream_t stream);

/*
 * Per-column sum and max of the same layouts: out[c] = reduction over
 * r < rows of x[r*ld + c], for c < cols (ld >= cols; ld == cols for a dense
 * matrix). out holds cols floats. Sums accumulate in float64 and round once
 * per column; max follows red_max_f32's rule. cols == 0 does nothing (out
 * may be NULL); rows == 0 stores 0.0f (sum) or -inf (max) in every out[c].
 * When there are few columns, the rows are cut into chunks whose partials
 * are added per column in a fixed order; a contiguous matrix may also be
 * read m rows at a time (one row of m * cols columns), and each column's m
 * partial columns are added the same way. Those partials live in a scratch
 * buffer of the stream that is grown on demand; an outgrown buffer is kept
 * until the process exits. Rows that do not start 16-byte aligned (of at
 * least 4 columns) are read as the aligned 16-byte vectors that cover them:
 * such a load may cover up to 3 elements before x[0] or after
 * x[(rows - 1) * ld + cols - 1], never outside the aligned vectors holding
 * those two; they, and the elements between rows, never enter a result.
 * Errors as for the row entry points.
 */
red_status red_cols_sum_f32(const float *x, size_t rows, size_t cols, size_t ld, float *out,
                            hipStream_t stream);
red_status red_cols_max_f32(const float *x, size_t rows, size_t cols, size_t ld, float *out,
                            hipStream_t stream);

/*
 * A fresh workspace for (current device, stream): allocates a new workspace
 * (zeroed on `stream`), which later calls on the stream and graphs captured
 * on it from now on use, and drops the stream's column scratch, which the
 * next column call on it allocates anew. The replaced buffers stay allocated
 * until the process exits, so graphs captured earlier keep working and may
 * run concurrently with graphs captured afterwards. Returns RED_ERR_CAPTURE
 * (allocating nothing) while the stream is being captured, RED_ERR_ALLOC if
 * the allocation fails.
 */
red_status red_stream_new_workspace(hipStream_t stream);

/* A static, human-readable name for a status code. */
const char *red_status_string(red_status status);

/*
 * The last hipError_t seen by a red_* call that returned RED_ERR_HIP,
 * RED_ERR_ALLOC or RED_ERR_NO_DEVICE on the calling thread (0 if none).
 */
int red_last_hip_error(void);

/* Library version string, e.g. "libred 0.1.0 gfx950". */
const char *red_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBRED_H_ */
