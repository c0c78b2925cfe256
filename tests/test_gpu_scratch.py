"""Library scratch memory, graphs and the read probe, on the GPU.

- Poison: the simulator page ("simt.py", section 3) fills shared memory with
  NaN so that a value read before it was written shows up. Here the library's
  own scratch (block partials, split-row partials, column partials) is
  filled with NaN, +inf, -inf or all-ones words before a call, and the call
  must still match the oracle: every partial it reads must be one it wrote.
- Graphs captured on one stream, with a fresh workspace between the
  captures, replay concurrently on two streams and match their eager
  results; a first call on a fresh stream during a capture on another
  stream allocates without disturbing that capture.
- The load-only read probe returns the xor of every word at every shape.
"""
import math
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
# 32-bit poison words: NaN (float32; float64 NaN as a pair), +inf, -inf (as
# float64 pairs: huge finite values of either sign), all ones (NaN, int64 -1).
POISON = (0x7FC00000, 0x7F800000, 0xFF800000, 0xFFFFFFFF)


def say(msg):
    print(f"[gpu-scratch] {msg}", flush=True)
    sys.stdout.flush()


def _dev(a, offset=0):
    dt = {np.float32: torch.float32, np.int32: torch.int32}[a.dtype.type]
    buf = torch.zeros(a.size + offset + 8, dtype=dt, device=DEV)
    v = buf[offset:offset + a.size]
    v.copy_(torch.from_numpy(np.ascontiguousarray(a.reshape(-1))))
    return v.view(a.shape) if a.ndim > 1 else v


def _sum_ok(got, S, A):
    return abs(float(got) - S) <= 1e-5 * A + 1e-6 and abs(float(got) - S) <= 2.0 ** -24 * abs(S) + 1e-12 * A


FLAT_SHAPES = (None, dict(combine=0), dict(block=256, blocks_per_cu=4, unroll=4, combine=1),
               dict(layout=0, block=1024, blocks_per_cu=1, unroll=4, prefetch=0, combine=0))


def test_poisoned_workspace_single_value_calls():
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    rng = np.random.default_rng(1201)
    a = rng.standard_normal((1 << 22) + 3).astype(np.float32)
    ai = rng.integers(-(2 ** 31), 2 ** 31, (1 << 22) + 1, dtype=np.int64).astype(np.int32)
    x, xi = _dev(a, 1), _dev(ai, 2)
    xh = x.to(torch.float16)
    xb = x.to(torch.bfloat16)
    xd = x.to(torch.float64)
    torch.cuda.synchronize()
    S, A = oracle.sum_f32(a)
    SI = oracle.sum_i32_i64(ai)
    M, MN = float(oracle.max_f32(a)), float(oracle.min_f32(a))
    AM, AN = oracle.argmax_f32(a), oracle.argmin_f32(a)
    bits_h = xh.cpu().view(torch.int16).numpy().view(np.uint16)
    bits_b = xb.cpu().view(torch.int16).numpy().view(np.uint16)
    SH, AH = oracle.sum_f16(bits_h)
    SB, AB = oracle.sum_bf16(bits_b)
    SD, AD = oracle.sum_f64(xd.cpu().numpy())
    SA, _ = oracle.sum_f32(np.abs(a))
    with torch.cuda.stream(s):
        for word in POISON:
            for pol in FLAT_SHAPES:
                say(f"poison {word:#010x} policy {pol}")
                checks = []
                for name, fn, arg in (("sum", rl.red_sum_f32, x), ("max", rl.red_max_f32, x),
                                      ("min", rl.red_min_f32, x), ("argmax", rl.red_argmax_f32, x),
                                      ("argmin", rl.red_argmin_f32, x), ("i32", rl.red_sum_i32_i64, xi),
                                      ("fused", rl.red_sum_max_f32, x), ("f16", rl.red_sum_f16_f32, xh),
                                      ("bf16", rl.red_sum_bf16_f32, xb), ("f64", rl.red_sum_f64, xd)):
                    rl.red_probe_fill_workspace(word, stream=s)
                    checks.append((name, fn(arg, policy=pol)))
                s.synchronize()
                got = {k: v.cpu() for k, v in checks}
                assert _sum_ok(got["sum"].item(), S, A), (word, pol)
                assert got["max"].item() == M and got["min"].item() == MN, (word, pol)
                assert int(got["argmax"].item()) == AM and int(got["argmin"].item()) == AN, (word, pol)
                assert int(got["i32"].item()) == SI, (word, pol)
                f3 = got["fused"].numpy()
                assert _sum_ok(f3[0], S, A) and f3[1] == M and _sum_ok(f3[2], SA, SA), (word, pol)
                assert abs(got["f16"].item() - SH) <= 1e-5 * AH + 1e-6, (word, pol)
                assert abs(got["bf16"].item() - SB) <= 1e-5 * AB + 1e-6, (word, pol)
                assert abs(got["f64"].item() - SD) <= 1e-12 * AD, (word, pol)
            say(f"poison {word:#010x}: allocation-free sum")
            rl.red_probe_fill_workspace(word, stream=s)
            o = rl.red_sum_f32_noalloc(x)
            s.synchronize()
            assert _sum_ok(o.item(), S, A)


def test_poisoned_scratch_rows_and_cols():
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    rng = np.random.default_rng(1202)
    cases = []
    for rows, cols in ((7, 1 << 20), (3, 70_001), (4099, 1024), (20_003, 7), (100, 1000), (5000, 33), (33, 4097)):
        a = rng.standard_normal((rows, cols)).astype(np.float32)
        cases.append((a, _dev(a, (rows + cols) % 4)))
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for a, x in cases:
            rows, cols = a.shape
            RS, RA = oracle.rows_sum_f32(a)
            RM = oracle.rows_max_f32(a)
            CS, CA = oracle.cols_sum_f32(a)
            CM = oracle.cols_max_f32(a)
            rl.red_cols_sum_f32(x)                 # the stream's column scratch exists from here on
            for word in POISON:
                say(f"poison {word:#010x} rows/cols {rows}x{cols}")
                outs = []
                for fn in (rl.red_rows_sum_f32, rl.red_rows_max_f32, rl.red_cols_sum_f32, rl.red_cols_max_f32):
                    rl.red_probe_fill_workspace(word, stream=s)
                    outs.append(fn(x))
                s.synchronize()
                rs, rm, cs, cm = (o.cpu().numpy() for o in outs)
                assert np.all(np.abs(rs.astype(np.float64) - RS) <= 1e-5 * RA + 1e-6), (word, rows, cols)
                assert np.array_equal(rm, RM), (word, rows, cols)
                assert np.all(np.abs(cs.astype(np.float64) - CS) <= 1e-5 * CA + 1e-6), (word, rows, cols)
                assert np.array_equal(cm, CM), (word, rows, cols)


def test_partials_overwrite_every_slot():
    # red_sum_f32_partials into a caller buffer full of NaN: each of the
    # `count` slots it reports must be written.
    rng = np.random.default_rng(1203)
    for n, pol in (((1 << 24) + 5, None), ((1 << 20) + 1, dict(block=256, blocks_per_cu=4, unroll=4)),
                   (1000, None), ((1 << 26) + 3, None)):
        say(f"partials into NaN n={n} policy={pol}")
        a = rng.standard_normal(n).astype(np.float32)
        x = _dev(a, 3)
        cap = rl.red_flat_grid(n, pol)
        buf = torch.full((cap + 16,), float("nan"), dtype=torch.float64, device=DEV)
        parts = rl.red_sum_f32_partials(x, partials=buf, policy=pol)
        torch.cuda.synchronize()
        p = parts.cpu().numpy()
        assert p.size == cap and not np.isnan(p).any(), (n, pol)
        assert np.isnan(buf[cap:].cpu().numpy()).all()              # nothing past the count
        S, A = oracle.sum_f32(a)
        assert abs(math.fsum(p.tolist()) - S) <= 1e-9 * A + 1e-12


def test_fill_refused_during_capture():
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        rl.red_probe_fill_workspace(0, stream=s)   # creates the workspace eagerly
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            with pytest.raises(rl.RedError) as ei:
                rl.red_probe_fill_workspace(0x7FC00000, stream=s)
        assert ei.value.status == rl.RED_ERR_CAPTURE
    torch.cuda.synchronize()


def test_graphs_with_own_workspaces_replay_concurrently():
    # Two graphs captured on one stream, with red_stream_new_workspace
    # between the captures, hold different buffers and may run at the same
    # time on different streams.
    rng = np.random.default_rng(1204)
    a1 = rng.standard_normal((1 << 23) + 3).astype(np.float32)
    a2 = rng.uniform(-1, 1, (1 << 23) + 11).astype(np.float32)
    m1 = rng.standard_normal((3000, 333)).astype(np.float32)
    m2 = rng.standard_normal((5000, 65)).astype(np.float32)
    x1, x2, y1, y2 = _dev(a1, 1), _dev(a2, 2), _dev(m1), _dev(m2)
    o1, o2 = torch.empty((), device=DEV), torch.empty((), device=DEV)
    c1, c2 = torch.empty(333, device=DEV), torch.empty(65, device=DEV)
    r1 = torch.empty(7, device=DEV)
    long_rows = _dev(rng.standard_normal((7, 1 << 18)).astype(np.float32))

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(cap):
        for x, y, o, c, with_rows in ((x1, y1, o1, c1, True), (x2, y2, o2, c2, False)):
            rl.red_stream_new_workspace(stream=cap)
            rl.red_sum_f32(x, out=o)               # warm: workspace and column scratch of this capture
            rl.red_cols_sum_f32(y, out=c)
            if with_rows:
                rl.red_rows_sum_f32(long_rows, out=r1)     # split rows: partials in the workspace
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                rl.red_sum_f32(x, out=o, policy=dict(combine=0))
                rl.red_sum_f32(x, out=o)
                rl.red_cols_sum_f32(y, out=c)
                if with_rows:
                    rl.red_rows_sum_f32(long_rows, out=r1)
            graphs.append(g)
    torch.cuda.synchronize()
    want = [rl.red_sum_f32(x1).item(), rl.red_sum_f32(x2).item()]
    want_c = [rl.red_cols_sum_f32(y1).clone(), rl.red_cols_sum_f32(y2).clone()]
    want_r = rl.red_rows_sum_f32(long_rows).clone()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for k in range(20):
        say(f"concurrent replay {k}")
        for t in (o1, o2, c1, c2, r1):
            t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            graphs[0].replay()
            graphs[0].replay()
        with torch.cuda.stream(sb):
            graphs[1].replay()
            graphs[1].replay()
        torch.cuda.synchronize()
        assert o1.item() == want[0] and o2.item() == want[1], k
        assert torch.equal(c1, want_c[0]) and torch.equal(c2, want_c[1]), k
        assert torch.equal(r1, want_r), k


def test_first_call_on_a_fresh_stream_during_another_capture():
    # PyTorch captures in global mode by default. A call on a stream that is
    # not being captured and has no workspace yet allocates one; it must
    # succeed and leave the other stream's capture intact.
    rng = np.random.default_rng(1205)
    a = rng.standard_normal((1 << 21) + 5).astype(np.float32)
    m = rng.standard_normal((2000, 100)).astype(np.float32)
    x, y = _dev(a, 1), _dev(m)
    S, A = oracle.sum_f32(a)
    CS, CA = oracle.cols_sum_f32(m)
    o_cap, o_fresh = torch.empty((), device=DEV), torch.empty((), device=DEV)
    c_fresh = torch.empty(100, device=DEV)
    cap, fresh = torch.cuda.Stream(), torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    fresh.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        rl.red_sum_f32(x, out=o_cap)
        torch.cuda.synchronize()
        want = o_cap.item()
        g = torch.cuda.CUDAGraph()
        say("capture on one stream, first calls on another")
        with torch.cuda.graph(g, stream=cap):
            rl.red_sum_f32(x, out=o_cap)
            rl.red_sum_f32(x, out=o_fresh, stream=fresh)
            rl.red_cols_sum_f32(y, out=c_fresh, stream=fresh)
    torch.cuda.synchronize()
    assert o_fresh.item() == want
    assert np.all(np.abs(c_fresh.cpu().numpy().astype(np.float64) - CS) <= 1e-5 * CA + 1e-6)
    for k in range(3):
        o_cap.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert o_cap.item() == want and _sum_ok(want, S, A), k


def _read_shapes():
    for block in (64, 256, 1024):
        for unroll in (4, 8, 16, 32):
            for layout in (0, 1, 2, 3):
                if block == 1024 and (unroll > 16 or (layout >= 2 and unroll > 8)):
                    continue
                for nt in (0, 1):
                    yield dict(block=block, blocks_per_cu=1 if block == 1024 else 3, unroll=unroll,
                               nontemporal=nt, layout=layout)


def test_read_ceiling_probe_every_shape():
    # Whole tiles, a partial tile and leftover vectors: the xor of all words
    # is exact whatever the order.
    rng = np.random.default_rng(1206)
    nvec = 64 * 32 * 37 + 64 * 5 + 17
    w = rng.integers(0, 2 ** 32, 4 * nvec, dtype=np.uint64).astype(np.uint32)
    want = int(np.bitwise_xor.reduce(w))
    x = torch.from_numpy(w.view(np.int32)).to(DEV)
    for shape in _read_shapes():
        say(f"read probe {shape}")
        sink = torch.zeros(1, dtype=torch.int32, device=DEV)
        rl.red_probe_read_ceiling(x, sink=sink, shape=shape)
        torch.cuda.synchronize()
        assert int(sink.item()) & 0xFFFFFFFF == want, shape
    say("read probe, default shape, 1 GiB workload")
    a = W.workload("sum_max_f32_2p28")
    x = torch.from_numpy(a).to(DEV)
    sink = rl.red_probe_read_ceiling(x)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == int(np.bitwise_xor.reduce(a.view(np.uint32)))
    with pytest.raises(rl.RedError):
        rl.red_probe_read_ceiling(x[1:5])          # not 16-byte aligned
    with pytest.raises(rl.RedError):
        rl.red_probe_read_ceiling(x, shape=dict(block=1024, unroll=32))


def test_copy_ceiling_probe_every_shape():
    # Whole tiles, a partial tile and leftover vectors, every compiled shape:
    # the copy must be exact, and nothing past the end may be written.
    rng = np.random.default_rng(1207)
    nvec = 64 * 16 * 23 + 64 * 3 + 11
    w = rng.integers(0, 2 ** 32, 4 * nvec, dtype=np.uint64).astype(np.uint32).view(np.int32)
    x = torch.from_numpy(w).to(DEV)
    for bpc in (1, 3):
        for unroll in (4, 8, 16):
            for nt in (0, 1):
                shape = dict(block=64, blocks_per_cu=bpc, unroll=unroll, nontemporal=nt, layout=2)
                say(f"copy probe {shape}")
                y = torch.full((4 * nvec + 8,), -7, dtype=torch.int32, device=DEV)
                rl.red_probe_copy_ceiling(x, y[: 4 * nvec], shape=shape)
                torch.cuda.synchronize()
                assert torch.equal(y[: 4 * nvec], x), shape
                assert torch.all(y[4 * nvec:] == -7), shape
    with pytest.raises(rl.RedError):
        rl.red_probe_copy_ceiling(x, torch.empty_like(x), shape=dict(layout=1))
