"""Pins for the CPU oracle: checks against facts fixed outside the oracle.

Each pin takes an `Oracle` (see oracle/__init__.py) and raises AssertionError
when the oracle disagrees with something the mathematics or the pages fix:
closed forms, the correctly rounded sum from Python's math.fsum (Shewchuk's
exact summation), brute force on tiny inputs, and the special cases of the
stated semantics. The pins are chosen so that each plausible slip in the
oracle (a dropped term, a wrong sign or index, the wrong accumulator width,
the wrong start value) fails at least one of them; test_oracle_mutations.py
plants such slips in copies of oracle.c and checks exactly that.
"""
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
U = 2.0 ** -53                       # unit roundoff of float64
BIG = float(np.float32(1e16))        # a float32 far above 2^53 / 2
I32_MIN = -(2 ** 31)
I32_MAX = 2 ** 31 - 1

# Non-power-of-two lengths around wave (64), block and vector boundaries.
LENGTHS = [1, 2, 3, 5, 7, 31, 33, 63, 65, 127, 129, 255, 257, 1000, 4097,
           65537, 1_000_003]


def _fsum(x):
    return math.fsum(np.asarray(x, dtype=np.float64).tolist())


def _mod7_closed(n):
    """sum_{i<n} (i mod 7): 21 per full cycle of 7, plus 0+1+..+(r-1)."""
    q, r = divmod(n, 7)
    return 21 * q + r * (r - 1) // 2


# ---------------------------------------------------------------- float sum

def pin_sum_arange_closed_form(o):
    # x_i = i is exact in float32 for i < 2^24; the sum n(n-1)/2 < 2^53.
    for n in LENGTHS:
        S, A = o.sum_f32(np.arange(n, dtype=np.float32))
        assert S == n * (n - 1) // 2, (n, S)
        assert A == n * (n - 1) // 2, (n, A)
        S, A = o.sum_f32(-np.arange(n, dtype=np.float32))
        assert S == -(n * (n - 1) // 2), (n, S)
        assert A == n * (n - 1) // 2, (n, A)


def pin_sum_all_ones(o):
    for n in LENGTHS:
        S, A = o.sum_f32(np.ones(n, np.float32))
        assert S == n and A == n, (n, S, A)


def pin_sum_compensation(o):
    # Plain float64 addition loses the small terms here; the exact sums are
    # 1, 2 and -3, and fsum agrees.
    cases = [([BIG, 1.0, -BIG], 1.0),
             ([1.0, BIG, 1.0, -BIG], 2.0),
             ([-1.0, -BIG, -2.0, BIG], -3.0)]
    for xs, want in cases:
        x = np.array(xs, np.float32)
        assert _fsum(x) == want
        S, A = o.sum_f32(x)
        assert S == want, (xs, S)
        # sum|x| is a plain float64 loop: within n roundings of itself.
        assert abs(A - _fsum(np.abs(x))) <= x.size * U * A, (xs, A)


def _random_sets():
    rng = np.random.default_rng(1234)
    sets = []
    # Mixed magnitudes 1e-8 .. 1e8 with random signs.
    mags = 10.0 ** rng.uniform(-8, 8, 200_000)
    sets.append((mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32))
    # Cancellation pairs (x, -x) shuffled in with small residue terms.
    base = rng.uniform(-1e6, 1e6, 50_000).astype(np.float32)
    res = rng.uniform(-1e-3, 1e-3, 1_000).astype(np.float32)
    pair = np.concatenate([base, -base, res])
    rng.shuffle(pair)
    sets.append(pair)
    # The wide mixture of the 1e9-element workload, at 10^6 elements.
    m = 1_000_000
    b = rng.uniform(-1, 1, m)
    pick = rng.random(m) < 0.01
    w = rng.uniform(-1e4, 1e4, m)
    sets.append(np.where(pick, w, b).astype(np.float32))
    # Tiny arrays.
    for n in (1, 2, 3, 4, 5, 17):
        sets.append(rng.standard_normal(n).astype(np.float32) * 1e3)
    return sets


_RANDOM_SETS = None


def pin_sum_matches_fsum(o):
    # Neumaier's error is about one rounding of |S| plus O(n u^2) sum|x|;
    # a plain float64 loop is off by O(sqrt(n) u) of the partial sums and
    # fails this bound on the sets above.
    global _RANDOM_SETS
    if _RANDOM_SETS is None:
        _RANDOM_SETS = _random_sets()
    for x in _RANDOM_SETS:
        want = _fsum(x)
        A_want = _fsum(np.abs(x))
        S, A = o.sum_f32(x)
        bound = 2 * U * abs(want) + 4 * x.size * U * U * A_want
        assert abs(S - want) <= bound, (x.size, S, want, bound)
        assert abs(A - A_want) <= x.size * U * A_want, (x.size, A, A_want)


def pin_sum_nonfinite(o):
    nan, inf = float("nan"), float("inf")
    f = lambda xs: o.sum_f32(np.array(xs, np.float32))[0]
    assert math.isnan(f([1.0, nan, 2.0]))
    assert math.isnan(f([inf, -inf]))
    assert math.isnan(f([-inf, 3.0, inf, 4.0]))
    assert f([1.0, inf, 2.0]) == inf
    assert f([-inf, 3.0, -inf]) == -inf
    assert f([inf, 5.0]) == inf
    # Sum|x| covers the finite inputs only.
    assert o.sum_f32(np.array([inf, -2.0, 3.0], np.float32))[1] == 5.0


MT_THREADS = (1, 2, 3, 8, 64)


def pin_sum_mt_closed_form(o):
    # The chunked form on several thread counts, including more threads than
    # elements (empty chunks): sum i = n(n-1)/2, exactly.
    for T in MT_THREADS:
        for n in LENGTHS:
            S, A = o.sum_f32_mt(np.arange(n, dtype=np.float32), T)
            assert S == n * (n - 1) // 2 and A == S, (T, n, S, A)


def pin_sum_mt_matches_fsum(o):
    # Each chunk keeps its (sum, correction) pair, accurate to second order,
    # and the pairs are added with the same compensated step, so the bound of
    # pin_sum_matches_fsum holds for every thread count; the single-threaded
    # and chunked results then also agree within 1e-15 * sum|x|.
    global _RANDOM_SETS
    if _RANDOM_SETS is None:
        _RANDOM_SETS = _random_sets()
    for x in _RANDOM_SETS:
        want = _fsum(x)
        A_want = _fsum(np.abs(x))
        S1, _ = o.sum_f32(x)
        for T in MT_THREADS:
            S, A = o.sum_f32_mt(x, T)
            bound = 2 * U * abs(want) + 4 * x.size * U * U * A_want
            assert abs(S - want) <= bound, (T, x.size, S, want, bound)
            assert abs(A - A_want) <= x.size * U * A_want, (T, x.size, A, A_want)
            assert abs(S - S1) <= 1e-15 * A_want, (T, x.size, S, S1)


def pin_sum_mt_nonfinite(o):
    nan, inf = float("nan"), float("inf")
    n = 1000
    for T in (2, 8):
        x = np.ones(n, np.float32)
        x[700] = nan                                   # in a late chunk
        assert math.isnan(o.sum_f32_mt(x, T)[0])
        x = np.ones(n, np.float32)
        x[10], x[990] = inf, -inf                      # opposite signs, different chunks
        assert math.isnan(o.sum_f32_mt(x, T)[0])
        x = np.ones(n, np.float32)
        x[990] = -inf
        S, A = o.sum_f32_mt(x, T)
        assert S == -inf and A == n - 1, (S, A)


def pin_sum_empty(o):
    assert o.sum_f32(np.zeros(0, np.float32)) == (0.0, 0.0)


def read_golden(name):
    """Parse `key=value` lines (comments start with #) of tests/golden/<name>."""
    rows = []
    with open(os.path.join(HERE, "golden", name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(dict(kv.split("=", 1) for kv in line.split()))
    return rows


def pin_sum_lesson_demo3(o):
    # The reduction lesson's own workload: x[i] = i mod 7 in float32 at the
    # full and quick sizes, checked against the closed form and the fixture.
    for row in read_golden("lesson_demo3_mod7.txt"):
        n, want = int(row["n"]), int(row["expected"])
        assert want == _mod7_closed(n)
        x = (np.arange(n) % 7).astype(np.float32)
        S, _ = o.sum_f32(x)
        assert S == want, (n, S, want)


# ---------------------------------------------------------------- int sum

def pin_int_closed_forms(o):
    for n in LENGTHS:
        assert o.sum_i32_i64(np.arange(n, dtype=np.int32)) == n * (n - 1) // 2
        assert o.sum_i32_i64(-np.ones(n, np.int32)) == -n
    # Sums far outside the int32 range.
    assert o.sum_i32_i64(np.full(1000, I32_MIN, np.int32)) == 1000 * I32_MIN
    assert o.sum_i32_i64(np.full(1001, I32_MAX, np.int32)) == 1001 * I32_MAX
    assert o.sum_i32_i64(np.array([I32_MAX, I32_MAX, I32_MIN], np.int32)) == I32_MAX - 1
    assert o.sum_i32_i64(np.zeros(0, np.int32)) == 0


def pin_int_brute_force(o):
    rng = np.random.default_rng(99)
    for n in (1, 2, 3, 63, 65, 1000, 100_003):
        x = rng.integers(I32_MIN, I32_MAX, n, dtype=np.int64, endpoint=True).astype(np.int32)
        assert o.sum_i32_i64(x) == sum(int(v) for v in x.tolist()), n


# ---------------------------------------------------------------- max

def pin_max_planted(o):
    rng = np.random.default_rng(7)
    for n in (1, 2, 3, 63, 64, 65, 257, 4097):
        for where in (0, n - 1, n // 2):
            x = rng.uniform(-100.0, -1.0, n).astype(np.float32)   # all negative
            x[where] = -0.5
            assert o.max_f32(x) == np.float32(-0.5), (n, where)
    assert o.max_f32(np.array([-np.inf, -5.0, -np.inf], np.float32)) == -5.0
    assert o.max_f32(np.array([-3.0, np.inf, 2.0], np.float32)) == np.inf
    assert o.max_f32(np.array([-np.inf], np.float32)) == -np.inf


def pin_max_nan_and_empty(o):
    nan = np.float32("nan")
    assert o.max_f32(np.array([nan, -7.0, -9.0], np.float32)) == -7.0
    assert o.max_f32(np.array([-7.0, nan, -9.0], np.float32)) == -7.0
    assert o.max_f32(np.array([-9.0, -7.0, nan], np.float32)) == -7.0
    assert o.max_f32(np.array([nan, nan], np.float32)) == -np.inf
    assert o.max_f32(np.zeros(0, np.float32)) == -np.inf


def pin_max_brute_force(o):
    rng = np.random.default_rng(8)
    for n in LENGTHS[:-1]:
        x = rng.standard_normal(n).astype(np.float32)
        assert o.max_f32(x) == max(x.tolist()), n


# ---------------------------------------------------------------- rows

def _rows_mod7_closed(r, cols):
    # sum over c < cols of (r + c) mod 7: full cycles give 21 each; the
    # remaining k terms run (r mod 7), (r mod 7) + 1, ... modulo 7.
    q, k = divmod(cols, 7)
    return 21 * q + sum((r + j) % 7 for j in range(k))


def pin_rows_closed_form(o):
    for rows, cols in ((1, 1), (3, 5), (9, 7), (13, 1000), (65, 257), (5, 4096)):
        x = ((np.arange(rows)[:, None] + np.arange(cols)[None, :]) % 7).astype(np.float32)
        S, A = o.rows_sum_f32(x)
        want = np.array([_rows_mod7_closed(r, cols) for r in range(rows)], np.float64)
        assert np.array_equal(S, want), (rows, cols)
        assert np.array_equal(A, want), (rows, cols)
        M = o.rows_max_f32(x)
        want_max = np.array([6.0 if cols >= 7 else float(max((r + c) % 7 for c in range(cols)))
                             for r in range(rows)], np.float32)
        assert np.array_equal(M, want_max), (rows, cols)


def pin_rows_brute_force(o):
    rng = np.random.default_rng(11)
    for rows, cols in ((1, 3), (4, 63), (7, 65), (33, 129), (16, 1001)):
        x = rng.standard_normal((rows, cols)).astype(np.float32)
        x[np.arange(rows), np.arange(rows) % cols] = 50.0 + np.arange(rows)  # planted max
        x[-1, -1] = 1000.0                                                   # last element
        S, A = o.rows_sum_f32(x)
        for r in range(rows):
            assert abs(S[r] - _fsum(x[r])) <= 2 * U * abs(_fsum(x[r])) + 1e-300, (rows, cols, r)
            assert abs(A[r] - _fsum(np.abs(x[r]))) <= cols * U * _fsum(np.abs(x[r]))
        assert np.array_equal(o.rows_max_f32(x), x.max(axis=1)), (rows, cols)


def pin_rows_degenerate(o):
    S, A = o.rows_sum_f32(np.zeros((4, 0), np.float32))
    assert np.array_equal(S, np.zeros(4)) and np.array_equal(A, np.zeros(4))
    assert np.array_equal(o.rows_max_f32(np.zeros((4, 0), np.float32)), np.full(4, -np.inf, np.float32))
    S, A = o.rows_sum_f32(np.zeros((0, 5), np.float32))
    assert S.size == 0 and A.size == 0


def pin_cols_brute_force(o):
    # Column reductions are the row reductions of the transpose; check them
    # against fsum and max over each column directly.
    rng = np.random.default_rng(12)
    for rows, cols in ((1, 1), (5, 3), (64, 7), (129, 65), (3, 1000)):
        x = rng.standard_normal((rows, cols)).astype(np.float32)
        x[(np.arange(cols) * 5) % rows, np.arange(cols)] = 77.0 + np.arange(cols)
        S, A = o.cols_sum_f32(x)
        for c in range(cols):
            col = x[:, c]
            assert abs(S[c] - _fsum(col)) <= 2 * U * abs(_fsum(col)) + 1e-300, (rows, cols, c)
            assert abs(A[c] - _fsum(np.abs(col))) <= rows * U * _fsum(np.abs(col))
        assert np.array_equal(o.cols_max_f32(x), x.max(axis=0)), (rows, cols)
    # (r + c) mod 7 is symmetric in r and c, so column sums follow the row
    # closed form with rows and columns swapped.
    x = ((np.arange(40)[:, None] + np.arange(9)[None, :]) % 7).astype(np.float32)
    S, _ = o.cols_sum_f32(x)
    assert np.array_equal(S, [_rows_mod7_closed(c, 40) for c in range(9)])


def pin_min_and_argext(o):
    rng = np.random.default_rng(13)
    nan, inf = np.float32("nan"), np.float32("inf")
    for n in (1, 2, 3, 63, 64, 65, 257, 4097):
        x = rng.uniform(1.0, 100.0, n).astype(np.float32)          # all positive
        for where in {0, n - 1, n // 2}:
            y = x.copy()
            y[where] = 0.5
            assert o.min_f32(y) == np.float32(0.5), (n, where)
            assert o.argmin_f32(y) == where, (n, where)
            z = -x
            z[where] = -0.5
            assert o.argmax_f32(z) == where, (n, where)
        vals = x.tolist()
        assert o.argmax_f32(x) == vals.index(max(vals))
        assert o.argmin_f32(x) == vals.index(min(vals))
    # Ties: the lowest index wins; -0 equals +0.
    t = np.array([1.0, 3.0, 2.0, 3.0, 3.0], np.float32)
    assert o.argmax_f32(t) == 1 and o.argmin_f32(t) == 0
    assert o.argmax_f32(np.array([-0.0, 0.0], np.float32)) == 0
    assert o.argmin_f32(np.array([0.0, -0.0], np.float32)) == 0
    # NaN never wins; no number at all gives -1 (and +inf for min).
    assert o.argmax_f32(np.array([nan, 2.0, nan, 5.0, nan], np.float32)) == 3
    assert o.argmin_f32(np.array([nan, 2.0, nan, 5.0], np.float32)) == 1
    assert o.argmax_f32(np.array([nan, nan], np.float32)) == -1
    assert o.argmax_f32(np.zeros(0, np.float32)) == -1
    assert o.min_f32(np.array([nan, nan], np.float32)) == inf
    assert o.min_f32(np.zeros(0, np.float32)) == inf
    # Infinities are numbers: all -inf has its argmax at index 0.
    assert o.argmax_f32(np.array([-inf, -inf], np.float32)) == 0
    assert o.argmin_f32(np.array([3.0, -inf, -inf], np.float32)) == 1


def pin_sum_f64(o):
    for n in LENGTHS:
        S, A = o.sum_f64(np.arange(n, dtype=np.float64))
        assert S == n * (n - 1) // 2 and A == S, n
    cases = [([1e300, 1.0, -1e300], 1.0), ([1.0, 2.0 ** 60, 1.0, -(2.0 ** 60)], 2.0)]
    for xs, want in cases:
        assert o.sum_f64(np.array(xs))[0] == want
    rng = np.random.default_rng(14)
    x = rng.standard_normal(100_000) * 10.0 ** rng.uniform(-10, 10, 100_000)
    want = _fsum(x)
    S, A = o.sum_f64(x)
    assert abs(S - want) <= 2 * U * abs(want) + 4 * x.size * U * U * _fsum(np.abs(x))
    assert np.isnan(o.sum_f64(np.array([1.0, np.nan]))[0])
    assert o.sum_f64(np.array([np.inf, 1.0]))[0] == np.inf


def pin_half_formats(o):
    # bfloat16 keeps float32's upper 16 bits; small integers are exact in both
    # 16-bit formats, so sums of them have closed forms.
    ints = np.arange(256, dtype=np.float32)
    bf = (ints.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bf.astype(np.uint32) << 16).view(np.float32), ints)
    assert o.sum_bf16(bf)[0] == 255 * 256 // 2
    hf = ints.astype(np.float16).view(np.uint16)
    assert o.sum_f16(hf)[0] == 255 * 256 // 2
    # Known bit patterns: bf16 0x3F80 = 1.0, 0xC000 = -2.0; f16 0x3C00 = 1.0,
    # 0x7BFF = 65504 (largest half), 0x0001 = 2^-24 (smallest subnormal).
    assert o.sum_bf16(np.array([0x3F80, 0xC000], np.uint16))[0] == -1.0
    assert o.sum_f16(np.array([0x3C00, 0x7BFF], np.uint16))[0] == 65505.0
    assert o.sum_f16(np.array([0x0001, 0x0001], np.uint16))[0] == 2.0 ** -23


PINS = [(name, fn) for name, fn in sorted(globals().items())
        if name.startswith("pin_") and callable(fn)]
