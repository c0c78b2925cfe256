"""The allocation-free float32 sum (red_sum_f32_noalloc), through the C ABI.

It must return exactly the bits of red_sum_f32 (same kernels, same launch
shapes, partials in a fixed device array instead of the stream's
workspace), and both must lie within |gpu - S| <= 1e-5 * sum|x| + 1e-6 of
the oracle's float64 compensated sum. Calls follow each other with smaller
inputs, so a combine that read a partial left by the previous call would
show.
"""
import ctypes
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected only with a GPU
    pytest.skip("no GPU visible", allow_module_level=True)

import reduction_libred_amd as rl  # noqa: E402

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _view(a, offset):
    buf = torch.full((a.size + offset + 8,), float("nan"), dtype=torch.float32, device=DEV)
    v = buf[offset:offset + a.size]
    v.copy_(torch.from_numpy(a))
    return v


def _check(x, a, S=None, A=None):
    got = rl.red_sum_f32_noalloc(x)
    ref = rl.red_sum_f32(x)
    torch.cuda.synchronize()
    if S is None:
        S, A = oracle.sum_f32(a)
    g, r = float(got.item()), float(ref.item())
    assert np.float32(g).tobytes() == np.float32(r).tobytes(), (a.size, g, r)
    assert oracle.sum_within_tolerance(g, S, A), (a.size, g, S, A)


def test_noalloc_two_calls_second_smaller():
    # The bench's workload (2^28 normal floats, seed 2) with its launch shape,
    # then smaller inputs with fewer blocks: each combine must read only
    # partials its own call wrote.
    say("noalloc 2^28 workload")
    a = W.workload("sum_max_f32_2p28")
    x = torch.from_numpy(a).to(DEV)
    _check(x, a)
    del x
    rng = np.random.default_rng(7)
    for n, off in (((1 << 22) + 5, 1), (100_003, 3), (5000, 2), (7, 0)):
        say(f"noalloc n={n} offset={off}")
        b = rng.uniform(-1, 1, n).astype(np.float32)
        _check(_view(b, off), b)


def test_noalloc_back_to_back_without_sync():
    # Two calls enqueued one after the other on one stream, the second on a
    # smaller input, synchronised only at the end: stream order alone keeps
    # them apart.
    rng = np.random.default_rng(11)
    a = rng.standard_normal((1 << 24) + 3).astype(np.float32)
    b = rng.standard_normal(300_001).astype(np.float32)
    xa, xb = _view(a, 1), _view(b, 2)
    say("noalloc back to back")
    oa = rl.red_sum_f32_noalloc(xa)
    ob = rl.red_sum_f32_noalloc(xb)
    torch.cuda.synchronize()
    ra, rb = rl.red_sum_f32(xa), rl.red_sum_f32(xb)
    torch.cuda.synchronize()
    assert oa.item() == ra.item() and ob.item() == rb.item()
    for got, arr in ((oa, a), (ob, b)):
        S, A = oracle.sum_f32(arr)
        assert oracle.sum_within_tolerance(float(got.item()), S, A)


def test_noalloc_exact_cases():
    # Small non-negative integers (the lesson's i mod 7) sum exactly in
    # float32 whatever the order: 21 per 7 elements, plus 0 + 1 + ... + (r-1).
    for n in (1, 1000, 1 << 20, (1 << 22) + 7):
        say(f"noalloc mod7 n={n}")
        r = n % 7
        got = rl.red_sum_f32_noalloc(_view(W.pattern_mod7(n), 1))
        torch.cuda.synchronize()
        assert got.item() == float(21 * (n // 7) + r * (r - 1) // 2)
    say("noalloc n=0")
    out = torch.full((), 5.0, device=DEV)
    rl.red_sum_f32_noalloc(torch.empty(0, device=DEV), out=out)
    torch.cuda.synchronize()
    assert out.item() == 0.0


def test_noalloc_argument_errors():
    x = torch.zeros(64, device=DEV)
    f = rl.lib().red_sum_f32_noalloc
    p = x.data_ptr()
    assert f(ctypes.c_void_p(p + 2), 4, ctypes.c_void_p(p + 128), None) == rl.RED_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(p), 16, ctypes.c_void_p(p + 8), None) == rl.RED_ERR_INVALID_ARG
    assert f(None, 4, ctypes.c_void_p(p), None) == rl.RED_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(p), 4, None, None) == rl.RED_ERR_INVALID_ARG
