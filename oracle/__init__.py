"""CPU oracle for the libred reductions (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library neither imports nor links it, and the
two share no code. The arithmetic lives in oracle.c (plain C, float64
compensated sum, exact int64 sum, scalar max loop); this module only loads
it and marshals numpy arrays.

Acceptance rule used with it (per row for the row-segmented forms): float
sums within |gpu - S| <= 1e-5 * sum|x_i| + 1e-6, integers bit-exact, max
exact by value.
"""
import ctypes
import math
import os

import numpy as np

from . import build as _build


def _as(x, dtype):
    a = np.asarray(x)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


class Oracle:
    """The oracle functions bound to one compiled copy of oracle.c."""

    def __init__(self, libpath):
        lib = ctypes.CDLL(libpath)
        P = ctypes.c_void_p
        Z = ctypes.c_size_t
        D = ctypes.POINTER(ctypes.c_double)
        lib.oracle_sum_f32.argtypes = [P, Z, D, D]
        lib.oracle_sum_f32.restype = None
        lib.oracle_sum_i32_i64.argtypes = [P, Z]
        lib.oracle_sum_i32_i64.restype = ctypes.c_int64
        lib.oracle_max_f32.argtypes = [P, Z]
        lib.oracle_max_f32.restype = ctypes.c_float
        lib.oracle_rows_sum_f32.argtypes = [P, Z, Z, P, P]
        lib.oracle_rows_sum_f32.restype = None
        lib.oracle_rows_max_f32.argtypes = [P, Z, Z, P]
        lib.oracle_rows_max_f32.restype = None
        lib.oracle_min_f32.argtypes = [P, Z]
        lib.oracle_min_f32.restype = ctypes.c_float
        lib.oracle_argmax_f32.argtypes = [P, Z]
        lib.oracle_argmax_f32.restype = ctypes.c_int64
        lib.oracle_argmin_f32.argtypes = [P, Z]
        lib.oracle_argmin_f32.restype = ctypes.c_int64
        lib.oracle_sum_f64.argtypes = [P, Z, D, D]
        lib.oracle_sum_f64.restype = None
        lib.oracle_sum_f32_mt.argtypes = [P, Z, ctypes.c_int, D, D]
        lib.oracle_sum_f32_mt.restype = ctypes.c_int
        self.lib = lib
        self.path = libpath

    def sum_f32(self, x):
        """Return (S, A): the float64 compensated sum of float32 x, and sum|x|."""
        a = _as(x, np.float32).ravel()
        s = ctypes.c_double()
        ab = ctypes.c_double()
        self.lib.oracle_sum_f32(a.ctypes.data, a.size, ctypes.byref(s), ctypes.byref(ab))
        return s.value, ab.value

    def sum_f32_mt(self, x, threads=None):
        """(S, A) like sum_f32, computed in `threads` contiguous chunks on as
        many host threads (default: all CPUs), chunk results added in order."""
        a = _as(x, np.float32).ravel()
        t = os.cpu_count() or 1 if threads is None else int(threads)
        s = ctypes.c_double()
        ab = ctypes.c_double()
        self.lib.oracle_sum_f32_mt(a.ctypes.data, a.size, t, ctypes.byref(s), ctypes.byref(ab))
        return s.value, ab.value

    def sum_i32_i64(self, x):
        """Return the exact int64 sum of int32 x as a Python int."""
        a = _as(x, np.int32).ravel()
        return int(self.lib.oracle_sum_i32_i64(a.ctypes.data, a.size))

    def max_f32(self, x):
        """Return the float32 maximum of x (NaN never wins; empty gives -inf)."""
        a = _as(x, np.float32).ravel()
        return np.float32(self.lib.oracle_max_f32(a.ctypes.data, a.size))

    def rows_sum_f32(self, x):
        """Per-row (S, A) of a 2-D float32 array: two float64 arrays."""
        a = _as(x, np.float32)
        if a.ndim != 2:
            raise ValueError("rows_sum_f32 needs a 2-D array")
        rows, cols = a.shape
        s = np.empty(rows, np.float64)
        ab = np.empty(rows, np.float64)
        self.lib.oracle_rows_sum_f32(a.ctypes.data, rows, cols, s.ctypes.data, ab.ctypes.data)
        return s, ab

    def rows_max_f32(self, x):
        """Per-row float32 maximum of a 2-D float32 array."""
        a = _as(x, np.float32)
        if a.ndim != 2:
            raise ValueError("rows_max_f32 needs a 2-D array")
        rows, cols = a.shape
        out = np.empty(rows, np.float32)
        self.lib.oracle_rows_max_f32(a.ctypes.data, rows, cols, out.ctypes.data)
        return out

    def min_f32(self, x):
        """float32 minimum (strictly-smaller rule from +inf; NaN never wins)."""
        a = _as(x, np.float32).ravel()
        return np.float32(self.lib.oracle_min_f32(a.ctypes.data, a.size))

    def argmax_f32(self, x):
        """Lowest index of the maximum among non-NaN elements, or -1."""
        a = _as(x, np.float32).ravel()
        return int(self.lib.oracle_argmax_f32(a.ctypes.data, a.size))

    def argmin_f32(self, x):
        """Lowest index of the minimum among non-NaN elements, or -1."""
        a = _as(x, np.float32).ravel()
        return int(self.lib.oracle_argmin_f32(a.ctypes.data, a.size))

    def sum_f64(self, x):
        """Return (S, A) for float64 x: compensated sum and sum|x|."""
        a = _as(x, np.float64).ravel()
        s = ctypes.c_double()
        ab = ctypes.c_double()
        self.lib.oracle_sum_f64(a.ctypes.data, a.size, ctypes.byref(s), ctypes.byref(ab))
        return s.value, ab.value

    def sum_bf16(self, bits):
        """(S, A) of bfloat16 values given as uint16 bit patterns: each value
        is the float32 whose upper 16 bits are the pattern (exact widening),
        then summed like float32 input."""
        b = np.ascontiguousarray(np.asarray(bits, np.uint16)).ravel()
        return self.sum_f32((b.astype(np.uint32) << 16).view(np.float32))

    def sum_f16(self, bits):
        """(S, A) of IEEE half values given as uint16 bit patterns, widened
        exactly to float32 (numpy's float16) and summed like float32 input."""
        b = np.ascontiguousarray(np.asarray(bits, np.uint16)).ravel()
        return self.sum_f32(b.view(np.float16).astype(np.float32))

    def cols_sum_f32(self, x):
        """Per-column (S, A) of a 2-D float32 array: the row oracle applied to
        the transposed array (sum along axis 0, by definition)."""
        return self.rows_sum_f32(np.ascontiguousarray(np.asarray(x, np.float32).T))

    def cols_max_f32(self, x):
        """Per-column float32 maximum (the row oracle on the transpose)."""
        return self.rows_max_f32(np.ascontiguousarray(np.asarray(x, np.float32).T))


_default = None


def default():
    """The oracle built from oracle.c in this directory (built if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def sum_f32(x):
    return default().sum_f32(x)


def sum_f32_mt(x, threads=None):
    return default().sum_f32_mt(x, threads)


def sum_i32_i64(x):
    return default().sum_i32_i64(x)


def max_f32(x):
    return default().max_f32(x)


def rows_sum_f32(x):
    return default().rows_sum_f32(x)


def rows_max_f32(x):
    return default().rows_max_f32(x)


def min_f32(x):
    return default().min_f32(x)


def argmax_f32(x):
    return default().argmax_f32(x)


def argmin_f32(x):
    return default().argmin_f32(x)


def sum_f64(x):
    return default().sum_f64(x)


def sum_bf16(bits):
    return default().sum_bf16(bits)


def sum_f16(bits):
    return default().sum_f16(bits)


def cols_sum_f32(x):
    return default().cols_sum_f32(x)


def cols_max_f32(x):
    return default().cols_max_f32(x)


def sum_within_tolerance(gpu, S, A):
    """The float-sum acceptance rule: |gpu - S| <= 1e-5*A + 1e-6 (in float64).

    A non-finite S must be matched exactly (NaN by NaN, an infinity by the
    same infinity)."""
    g = float(gpu)
    if math.isnan(S):
        return math.isnan(g)
    if math.isinf(S):
        return g == S
    return abs(g - S) <= 1e-5 * A + 1e-6


def max_equal(gpu, expect):
    """Max acceptance: equal by value (so -0 == +0); -inf must match -inf."""
    return float(gpu) == float(expect)
