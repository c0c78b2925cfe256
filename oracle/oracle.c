/*
 * oracle.c -- CPU oracle for the libred reductions.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this code. The GPU library does not
 * include, link or call it, and it shares no source with the GPU library.
 *
 * It is plain and slow on purpose (single-threaded, except for one
 * chunked form of the float sum that splits the same computation over host
 * threads). Each function states the definition it computes and the passage
 * of the pages it follows:
 *
 *   [lesson] "03_shared_memory_sync_reduction.py -- shared memory, banks,
 *            synchronisation and parallel reduction" (CS349E prereq P2),
 *            demo 3 (parallel reduction): reduce n float32 values to one sum.
 *            The page checks its GPU-style result against the float64 sum of
 *            the same float32 inputs.
 *   [simt]   "simt.py -- a SIMT GPU simulator in Python" (CMU 11-868
 *            lecture 2), section 2 (device memory), DeviceArray.atomic_max:
 *            the stored value is replaced only when the new value is strictly
 *            greater.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared, never with -ffast-math (that would
 * let the compiler delete the compensation term of the compensated sum).
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>

/*
 * Sum of n float32 values, as the real sum of the inputs.
 *
 * Definition: S = x_0 + x_1 + ... + x_{n-1} over the reals ([lesson], demo 3,
 * where the expected value is the float64 sum of the float32 inputs).
 * Evaluation: each input is widened to double (exactly) and added with
 * Neumaier's compensated summation (Neumaier 1974, "Rundungsfehleranalyse
 * einiger Verfahren zur Summation endlicher Summen"): a running sum s and a
 * running correction c that collects the low-order bits each addition
 * loses. Whichever operand of s + x is larger in magnitude is the one whose
 * low bits survive, so the lost part is recovered from the other one.
 * The error of s + c is at most about one rounding of |S| plus a term of
 * order n * eps^2 * sum|x_i|, far below the tolerance this sum is used for.
 *
 * Non-finite inputs follow IEEE arithmetic on the real sum: any NaN, or both
 * +inf and -inf, gives NaN; otherwise an infinity of one sign gives that
 * infinity. They are counted apart, since the compensation term itself
 * would turn into NaN on an infinity.
 *
 * *abs_sum receives sum |x_i| over the finite inputs in plain double
 * arithmetic (used only to scale a tolerance). n == 0 gives 0 and 0.
 */
typedef struct {
    double s, c, a;              /* running sum, correction, sum of |x| */
    int saw_nan, saw_pinf, saw_ninf;
} neumaier_t;

static void nm_init(neumaier_t *st)
{
    st->s = st->c = st->a = 0.0;
    st->saw_nan = st->saw_pinf = st->saw_ninf = 0;
}

/* One compensated addition of a finite v to (s, c). */
static void nm_step(neumaier_t *st, double v)
{
    double t = st->s + v;
    if (fabs(st->s) >= fabs(v))
        st->c += (st->s - t) + v;   /* v's low bits were lost */
    else
        st->c += (v - t) + st->s;   /* s's low bits were lost */
    st->s = t;
}

static void nm_add(neumaier_t *st, double v)
{
    if (isnan(v)) { st->saw_nan = 1; return; }
    if (isinf(v)) {
        if (v > 0) st->saw_pinf = 1; else st->saw_ninf = 1;
        return;
    }
    st->a += fabs(v);
    nm_step(st, v);
}

static void nm_result(const neumaier_t *st, double *sum, double *abs_sum)
{
    if (abs_sum) *abs_sum = st->a;
    if (st->saw_nan || (st->saw_pinf && st->saw_ninf)) *sum = NAN;
    else if (st->saw_pinf) *sum = INFINITY;
    else if (st->saw_ninf) *sum = -INFINITY;
    else *sum = st->s + st->c;
}

static void neumaier_f32(const float *x, size_t n, double *sum, double *abs_sum)
{
    neumaier_t st;
    size_t i;
    nm_init(&st);
    for (i = 0; i < n; ++i)
        nm_add(&st, (double)x[i]);   /* float32 widens to double exactly */
    nm_result(&st, sum, abs_sum);
}

void oracle_sum_f32(const float *x, size_t n, double *sum, double *abs_sum)
{
    neumaier_f32(x, n, sum, abs_sum);
}

/*
 * The same sum on several host threads. x is cut into `threads` contiguous
 * chunks, chunk k being x[floor(k*n/T) .. floor((k+1)*n/T)); each thread runs
 * the compensated summation above over its chunk, and the chunks' running
 * sums and corrections are then added in chunk order with the same
 * compensated step (sum|x| and the non-finite flags are simply combined).
 * The result depends only on n and T, not on thread timing, and its error is
 * of the same order as the single-threaded form's. threads < 1 means 1;
 * more than 256 are capped at 256.
 */
typedef struct {
    const float *x;
    size_t n;
    neumaier_t st;
} nm_chunk_t;

static void *nm_chunk_run(void *arg)
{
    nm_chunk_t *ch = (nm_chunk_t *)arg;
    neumaier_t st;   /* thread-local: the chunk records sit side by side */
    size_t i;
    nm_init(&st);
    for (i = 0; i < ch->n; ++i)
        nm_add(&st, (double)ch->x[i]);
    ch->st = st;
    return NULL;
}

int oracle_sum_f32_mt(const float *x, size_t n, int threads, double *sum, double *abs_sum)
{
    nm_chunk_t ch[256];
    pthread_t tid[256];
    int started[256];
    neumaier_t tot;
    int T, k;
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    T = threads;
    for (k = 0; k < T; ++k) {
        size_t lo = (size_t)k * n / (size_t)T, hi = (size_t)(k + 1) * n / (size_t)T;
        ch[k].x = x + lo;
        ch[k].n = hi - lo;
        started[k] = pthread_create(&tid[k], NULL, nm_chunk_run, &ch[k]) == 0;
        if (!started[k]) nm_chunk_run(&ch[k]);   /* no thread: run it here */
    }
    nm_init(&tot);
    for (k = 0; k < T; ++k) {
        if (started[k]) pthread_join(tid[k], NULL);
        tot.saw_nan |= ch[k].st.saw_nan;
        tot.saw_pinf |= ch[k].st.saw_pinf;
        tot.saw_ninf |= ch[k].st.saw_ninf;
        tot.a += ch[k].st.a;
        nm_step(&tot, ch[k].st.s);
        nm_step(&tot, ch[k].st.c);
    }
    nm_result(&tot, sum, abs_sum);
    return T;
}

/*
 * Sum of n int32 values, exact, as a 64-bit integer ([lesson], demo 3's
 * reduction applied to integers). Accumulated in uint64_t so that a sum
 * outside the int64 range wraps modulo 2^64 instead of being undefined;
 * with |x_i| <= 2^31 that cannot happen for n < 2^32.
 */
int64_t oracle_sum_i32_i64(const int32_t *x, size_t n)
{
    uint64_t s = 0;
    size_t i;
    for (i = 0; i < n; ++i)
        s += (uint64_t)(int64_t)x[i];
    return (int64_t)s;
}

/*
 * Maximum of n float32 values ([simt], section 2, DeviceArray.atomic_max:
 * the running value is replaced only by a strictly greater one). Start from
 * -inf. A NaN compares false, so it never replaces the running maximum; an
 * empty or all-NaN input gives -inf. Ties keep the earlier value.
 */
float oracle_max_f32(const float *x, size_t n)
{
    float m = -INFINITY;
    size_t i;
    for (i = 0; i < n; ++i)
        if (x[i] > m) m = x[i];
    return m;
}

/*
 * Minimum of n float32 values: the mirror of oracle_max_f32. The running
 * value is replaced only by a strictly smaller one, starting from +inf; a NaN
 * never wins; empty or all-NaN gives +inf.
 */
float oracle_min_f32(const float *x, size_t n)
{
    float m = INFINITY;
    size_t i;
    for (i = 0; i < n; ++i)
        if (x[i] < m) m = x[i];
    return m;
}

/*
 * Index of the maximum (sign = +1) or minimum (sign = -1) of n float32
 * values: the lowest index i whose x[i] is not NaN and is >= (resp. <=) every
 * other non-NaN element. -1 when no element is a number (n == 0 included).
 * Scanning upward and replacing only on a strictly better value keeps the
 * first of equal extremes; -0 and +0 are equal.
 */
static int64_t arg_extreme(const float *x, size_t n, int sign)
{
    int64_t best = -1;
    float m = 0.0f;
    size_t i;
    for (i = 0; i < n; ++i) {
        if (isnan(x[i])) continue;
        if (best < 0 || (sign > 0 ? x[i] > m : x[i] < m)) {
            m = x[i];
            best = (int64_t)i;
        }
    }
    return best;
}

int64_t oracle_argmax_f32(const float *x, size_t n) { return arg_extreme(x, n, +1); }
int64_t oracle_argmin_f32(const float *x, size_t n) { return arg_extreme(x, n, -1); }

/*
 * Sum of n float64 values with the same compensated summation and
 * non-finite rules as oracle_sum_f32 (the inputs are already doubles).
 */
void oracle_sum_f64(const double *x, size_t n, double *sum, double *abs_sum)
{
    neumaier_t st;
    size_t k;
    nm_init(&st);
    for (k = 0; k < n; ++k)
        nm_add(&st, x[k]);
    nm_result(&st, sum, abs_sum);
}

/*
 * Row-segmented forms: x is rows x cols, row-major and contiguous (row r is
 * x[r*cols .. r*cols + cols)). Each row is reduced on its own with the
 * definitions above ([lesson], demo 3: one output per segment). rows == 0
 * writes nothing; cols == 0 gives the empty-row values (0, 0, -inf).
 */
void oracle_rows_sum_f32(const float *x, size_t rows, size_t cols,
                         double *sum, double *abs_sum)
{
    size_t r;
    for (r = 0; r < rows; ++r)
        neumaier_f32(x + r * cols, cols, &sum[r], abs_sum ? &abs_sum[r] : NULL);
}

void oracle_rows_max_f32(const float *x, size_t rows, size_t cols, float *out)
{
    size_t r;
    for (r = 0; r < rows; ++r)
        out[r] = oracle_max_f32(x + r * cols, cols);
}
