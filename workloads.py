"""Seeded synthetic inputs for the reduction workloads.

This module only draws and lays out input arrays. It holds none of the
reduction arithmetic, and it is the one piece of code that both the CPU
oracle's tests and the GPU path's tests and benchmark use.

Every random array comes from numpy's PCG64 in fixed chunks of CHUNK = 2^24
elements: chunk k (elements [k*CHUNK, (k+1)*CHUNK)) is drawn by
`default_rng(SeedSequence(seed, spawn_key=(k,)))`, so the bytes depend only on
(kind, n, seed), and chunks can be filled by parallel threads. The five named
workloads:

  sum_f32_2p20         2^20 float32, uniform[-1, 1), seed 0
  sum_i32_2p24         2^24 int32, integers in [-1000, 1000], seed 1
  sum_max_f32_2p28     2^28 float32 (1 GiB), standard normal, seed 2
  rows_f32_65536x4096  65536 x 4096 float32 row-major, uniform[0, 1), seed 3
  sum_f32_1e9p7        1,000,000,007 float32, per element: with probability
                       0.01 uniform[-1e4, 1e4), else uniform[-1, 1), seed 4

The structured patterns at the end are deterministic, not random; the
reduction lesson's own workload (the value i mod 7 at index i) is one.
"""
import concurrent.futures as cf
import os

import numpy as np

CHUNK = 1 << 24

# name -> (kind, shape, seed, description)
WORKLOADS = {
    "sum_f32_2p20": ("uniform_pm1", (1 << 20,), 0,
                     "float32 sum of 2^20 elements, uniform[-1,1), seed 0"),
    "sum_i32_2p24": ("int_pm1000", (1 << 24,), 1,
                     "int32 sum of 2^24 elements into int64, integers in [-1000,1000], seed 1"),
    "sum_max_f32_2p28": ("normal", (1 << 28,), 2,
                         "float32 sum and max of 2^28 elements (1 GiB), normal(0,1), seed 2"),
    "rows_f32_65536x4096": ("uniform01", (65536, 4096), 3,
                            "row sum and row max of 65536 x 4096 float32 row-major, uniform[0,1), seed 3"),
    "sum_f32_1e9p7": ("mixture", (1_000_000_007,), 4,
                      "float32 sum of 1,000,000,007 elements, 99% uniform[-1,1) + 1% uniform[-1e4,1e4), seed 4"),
}

DTYPES = {
    "uniform_pm1": np.float32,
    "int_pm1000": np.int32,
    "normal": np.float32,
    "uniform01": np.float32,
    "mixture": np.float32,
}


def _fill_chunk(kind, rng, out):
    m = out.size
    if kind == "uniform_pm1":
        out[:] = rng.uniform(-1.0, 1.0, m)
    elif kind == "int_pm1000":
        out[:] = rng.integers(-1000, 1001, m, dtype=np.int32)
    elif kind == "normal":
        rng.standard_normal(m, dtype=np.float32, out=out)
    elif kind == "uniform01":
        rng.random(m, dtype=np.float32, out=out)
    elif kind == "mixture":
        base = rng.uniform(-1.0, 1.0, m)
        pick = rng.random(m) < 0.01
        wide = rng.uniform(-1.0e4, 1.0e4, m)
        out[:] = np.where(pick, wide, base)
    else:
        raise ValueError(f"unknown kind {kind!r}")


def chunk_rng(seed, k):
    """The generator that draws chunk k of a workload with this seed."""
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(k,)))


def make(kind, n, seed, out=None, progress=None, threads=None):
    """Draw n elements of distribution `kind` for `seed`, chunk by chunk.

    Chunk k always holds the same values for a given seed, so
    make(kind, n, seed)[:m] equals make(kind, m, seed) whenever m is a
    multiple of CHUNK. `out` may be a preallocated array of the kind's dtype
    and n elements. `progress`, if given, is called with each finished chunk
    count. `threads` defaults to min(16, cpu count).
    """
    dtype = DTYPES[kind]
    if out is None:
        out = np.empty(n, dtype=dtype)
    if out.dtype != dtype or out.size != n:
        raise ValueError("out has the wrong dtype or size")
    flat = out.reshape(-1)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(k):
        lo = k * CHUNK
        _fill_chunk(kind, chunk_rng(seed, k), flat[lo:min(n, lo + CHUNK)])
        return k

    threads = threads or min(16, os.cpu_count() or 1)
    if nchunks <= 1 or threads <= 1:
        for k in range(nchunks):
            fill(k)
            if progress is not None:
                progress(k + 1)
    else:
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            for done, _ in enumerate(ex.map(fill, range(nchunks)), 1):
                if progress is not None:
                    progress(done)
    return out


def workload(name, progress=None):
    """The named workload's full input array (shape and dtype as listed)."""
    kind, shape, seed, _ = WORKLOADS[name]
    n = int(np.prod(shape))
    return make(kind, n, seed, progress=progress).reshape(shape)


def describe(name):
    kind, shape, seed, desc = WORKLOADS[name]
    return {"kind": kind, "shape": list(shape), "seed": seed,
            "dtype": np.dtype(DTYPES[kind]).name, "description": desc,
            "chunk": CHUNK}


# --- deterministic patterns -------------------------------------------------

def pattern_mod7(n, dtype=np.float32):
    """x[i] = i mod 7, the reduction lesson's input (demo 3)."""
    return (np.arange(n, dtype=np.int64) % 7).astype(dtype)


def pattern_every(n, every, dtype=np.float32):
    """x[i] = 1 where i is a multiple of `every`, else 0."""
    x = np.zeros(n, dtype=dtype)
    x[::every] = 1
    return x


def pattern_tags(n, positions, dtype=np.float32):
    """x[p_k] = 2^k for the k-th listed position (all distinct), else 0.

    With fewer than 24 tags every partial sum is exact in float32, and the
    bits of the total say exactly which tagged elements were counted."""
    positions = list(positions)
    if len(set(positions)) != len(positions):
        raise ValueError("tag positions must be distinct")
    x = np.zeros(n, dtype=dtype)
    for k, p in enumerate(positions):
        x[p] = 2.0 ** k
    return x


def pattern_rows_mod7(rows, cols, dtype=np.float32):
    """x[r, c] = (r + c) mod 7."""
    r = np.arange(rows, dtype=np.int64)[:, None]
    c = np.arange(cols, dtype=np.int64)[None, :]
    return ((r + c) % 7).astype(dtype)
