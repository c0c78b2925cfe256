"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Float sums must lie within |gpu - S| <= 1e-5 * sum|x| + 1e-6 of the oracle's
float64 compensated sum (per row for the row sums); integer sums and every
max must match exactly. The sums the headers promise to accumulate in
float64 and round once to float32 are also held to that promise:
|gpu - S| <= 2^-24 * |S| + 1e-12 * sum|x| (one float32 rounding of the
result, plus float64 rounding along chains of at most a few thousand
additions: h * 2^-53 < 1e-12 for h < 9000). A float32 accumulator anywhere
on such a path would break it. Inputs are the seeded workloads of workloads.py and
deterministic patterns. Views into larger buffers give misaligned heads and
ragged tails, and the elements just outside each view hold NaN (or +inf for
max), so reading one element too many changes the answer.
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
RAGGED = [1, 2, 3, 4, 5, 7, 31, 63, 64, 65, 127, 255, 256, 257, 1023, 1024, 1025,
          4095, 4096, 4097, 65535, 65537, 1_000_003, (1 << 22) + 5]
OFFSETS = [0, 1, 2, 3]


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def device_view(a, offset=0, guard=float("nan")):
    """Copy numpy array `a` into a fresh device buffer at element `offset`
    and return the view; elements before and after it hold `guard`."""
    dt = {np.float32: torch.float32, np.int32: torch.int32}[a.dtype.type]
    n = a.size
    buf = torch.empty(n + offset + 8, dtype=dt, device=DEV)
    buf.fill_(guard if dt == torch.float32 else -(2 ** 31))
    view = buf[offset:offset + n]
    view.copy_(torch.from_numpy(np.ascontiguousarray(a.reshape(-1))))
    return view.view(a.shape) if a.ndim > 1 else view


def gpu_sum(x, **kw):
    out = rl.red_sum_f32(x, **kw)
    torch.cuda.synchronize()
    return float(out.item())


U32 = 2.0 ** -24          # unit roundoff of float32
F64_CHAIN = 1e-12         # float64 accumulation error per unit of sum|x|


def f64_contract_ok(got, S, A):
    """|got - S| <= 2^-24 |S| + 1e-12 A elementwise (finite S), plus the
    size of a float32 subnormal step."""
    got = np.asarray(got, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    return bool(np.all(np.abs(got - S) <= U32 * np.abs(S) + F64_CHAIN * A + 2.0 ** -149))


def sums_ok(got, S, A):
    """Both bars for finite sums accumulated in float64: the 1e-5 acceptance
    bound and the one-rounding contract."""
    g = np.asarray(got, dtype=np.float64)
    return bool(np.all(np.abs(g - S) <= 1e-5 * A + 1e-6)) and f64_contract_ok(g, S, A)


def assert_sum_ok(got, a):
    S, A = oracle.sum_f32(a)
    assert oracle.sum_within_tolerance(got, S, A), (got, S, A, a.size)
    if math.isfinite(S):
        assert f64_contract_ok(got, S, A), ("float64 contract", got, S, A, a.size)


# ----------------------------------------------------------------- f32 sum

@pytest.mark.parametrize("offset", OFFSETS)
def test_sum_f32_ragged_random(offset):
    rng = np.random.default_rng(100 + offset)
    for n in RAGGED:
        say(f"sum_f32 n={n} offset={offset}")
        a = rng.uniform(-1, 1, n).astype(np.float32)
        x = device_view(a, offset)
        got = gpu_sum(x)
        assert_sum_ok(got, a)
        assert gpu_sum(x) == got            # bitwise run-to-run


def test_sum_f32_empty():
    say("sum_f32 n=0")
    out = torch.full((), 123.0, device=DEV)
    rl.red_sum_f32(torch.empty(0, device=DEV), out=out)
    torch.cuda.synchronize()
    assert out.item() == 0.0


def test_sum_f32_lesson_mod7_exact():
    # The lesson's workload: with small non-negative integers every partial
    # sum is exact in float32, so any order gives the exact total.
    for row in __import__("oracle_pins").read_golden("lesson_demo3_mod7.txt"):
        n, want = int(row["n"]), int(row["expected"])
        say(f"sum_f32 mod7 n={n}")
        assert gpu_sum(device_view(W.pattern_mod7(n))) == want


@pytest.mark.parametrize("n", [1 << 20, (1 << 24) + 3, 100_000_007])
def test_sum_f32_sparse_ones_exact(n):
    say(f"sum_f32 sparse ones n={n}")
    a = W.pattern_every(n, 64)
    assert gpu_sum(device_view(a, 1)) == float(len(range(0, n, 64)))


@pytest.mark.parametrize("offset", OFFSETS)
def test_sum_f32_tags_exact(offset):
    # Tags 2^k at the head, the tail and around vector, wave, block and grid
    # boundaries; each must be counted exactly once.
    n = (1 << 22) + 7
    pos = sorted({0, 1, 2, 3, 4, 5, 63, 64, 1023, 1024, 4095, 4096, 4097,
                  (1 << 20) - 1, 1 << 20, n - 4, n - 3, n - 2, n - 1, n // 2, 12345})
    say(f"sum_f32 tags n={n} offset={offset}")
    a = W.pattern_tags(n, pos)
    assert gpu_sum(device_view(a, offset)) == float(2 ** len(pos) - 1)


def test_sum_f32_nonfinite():
    cases = [([1.0, float("nan"), 2.0], "nan"), ([float("inf"), float("-inf")], "nan"),
             ([1.0, float("inf")], float("inf")), ([-3.0, float("-inf")], float("-inf"))]
    for xs, want in cases:
        for n_pad in (0, 5000):
            a = np.concatenate([np.zeros(n_pad, np.float32), np.array(xs, np.float32)])
            say(f"sum_f32 nonfinite {xs} pad={n_pad}")
            got = gpu_sum(device_view(a, 0, guard=0.0))
            assert (math.isnan(got) if want == "nan" else got == want), (xs, got)


def all_flat_policies(bpcs=(1, 4)):
    """Every compiled launch shape of the single-value kernels."""
    shapes = []
    for bpc in bpcs:
        for nt in (0, 1):
            for combine in (0, 1):
                for block in (256, 1024):
                    for unroll in (1, 4, 8):
                        shapes.append(dict(block=block, blocks_per_cu=bpc, unroll=unroll, nontemporal=nt,
                                           layout=0, prefetch=0, combine=combine))
                for block in (64, 256, 1024):
                    for unroll in (4, 8, 16):
                        for pf in (0, 1):
                            shapes.append(dict(block=block, blocks_per_cu=bpc, unroll=unroll,
                                               nontemporal=nt, layout=1, prefetch=pf, combine=combine))
    return shapes


def test_sum_f32_all_policies_agree():
    # Sizes that leave whole tiles, a partial tile and a ragged tail.
    for n, off in (((1 << 21) + 3, 2), ((1 << 23) + 4099, 1)):
        a = W.make("normal", n, 77)
        x = device_view(a, off)
        S, A = oracle.sum_f32(a)
        for p in all_flat_policies():
            say(f"sum_f32 n={n} policy {p}")
            got = gpu_sum(x, policy=p)
            assert oracle.sum_within_tolerance(got, S, A), (p, got, S)
            assert f64_contract_ok(got, S, A), ("float64 contract", p, got, S)


def test_sum_f32_partials():
    # Steps 1-5 alone: one float64 partial per block; their sum is the sum.
    for n, off in ((1, 0), (1000, 1), ((1 << 20) + 3, 2), ((1 << 24) + 5, 3), ((1 << 26) + 77, 1)):
        a = W.make("normal", n, 500 + off)
        x = device_view(a, off)
        S, A = oracle.sum_f32(a)
        for p in (None, dict(layout=0, block=256, blocks_per_cu=1, unroll=8, prefetch=0)):
            say(f"sum_f32_partials n={n} policy={p}")
            parts = rl.red_sum_f32_partials(x, policy=p)
            torch.cuda.synchronize()
            assert parts.numel() == rl.red_flat_grid(n, p)
            got = math.fsum(parts.cpu().numpy().tolist())
            assert abs(got - S) <= 1e-9 * A + 1e-12, (n, p, got, S)


def test_sum_f32_two_streams():
    # Calls on different streams use different workspaces and may overlap.
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    a1 = W.make("normal", 1 << 22, 5)
    a2 = W.make("uniform_pm1", (1 << 22) + 1, 6)
    x1, x2 = device_view(a1), device_view(a2)
    torch.cuda.synchronize()
    o1 = torch.empty(64, device=DEV)
    o2 = torch.empty(64, device=DEV)
    say("sum_f32 two streams x64")
    for k in range(64):
        rl.red_sum_f32(x1, out=o1[k], stream=s1)
        rl.red_sum_f32(x2, out=o2[k], stream=s2)
    torch.cuda.synchronize()
    for a, o in ((a1, o1), (a2, o2)):
        vals = o.cpu().numpy()
        assert np.all(vals == vals[0])
        assert_sum_ok(vals[0], a)


# ----------------------------------------------------------------- i32 -> i64

@pytest.mark.parametrize("offset", OFFSETS)
def test_sum_i32_ragged_random(offset):
    rng = np.random.default_rng(200 + offset)
    for n in RAGGED:
        say(f"sum_i32 n={n} offset={offset}")
        a = rng.integers(-(2 ** 31), 2 ** 31, n, dtype=np.int64).astype(np.int32)
        out = rl.red_sum_i32_i64(device_view(a, offset))
        torch.cuda.synchronize()
        assert int(out.item()) == oracle.sum_i32_i64(a), n


def test_sum_i32_closed_forms_and_empty():
    n = 1 << 24
    say("sum_i32 arange 2^24")
    out = rl.red_sum_i32_i64(torch.arange(n, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert int(out.item()) == n * (n - 1) // 2
    say("sum_i32 INT32_MIN x (2^20+3)")
    m = (1 << 20) + 3
    out = rl.red_sum_i32_i64(torch.full((m,), -(2 ** 31), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert int(out.item()) == m * -(2 ** 31)
    say("sum_i32 n=0")
    out = torch.full((), 5, dtype=torch.int64, device=DEV)
    rl.red_sum_i32_i64(torch.empty(0, dtype=torch.int32, device=DEV), out=out)
    torch.cuda.synchronize()
    assert int(out.item()) == 0


# ----------------------------------------------------------------- max

@pytest.mark.parametrize("offset", OFFSETS)
def test_max_f32_planted(offset):
    rng = np.random.default_rng(300 + offset)
    for n in RAGGED:
        for where in {0, n - 1, n // 2, min(n - 1, 3)}:
            say(f"max_f32 n={n} offset={offset} at={where}")
            a = rng.uniform(-100.0, -1.0, n).astype(np.float32)    # all negative
            a[where] = -0.25
            out = rl.red_max_f32(device_view(a, offset, guard=float("inf")))
            torch.cuda.synchronize()
            assert out.item() == -0.25 == float(oracle.max_f32(a)), (n, where)


def test_max_f32_nan_inf_empty():
    nan, inf = float("nan"), float("inf")
    cases = [([nan, -7.0, -9.0], -7.0), ([-9.0, nan], -9.0), ([nan, nan], -inf),
             ([-inf, -inf], -inf), ([-3.0, inf], inf), ([0.0, -0.0], 0.0)]
    for xs, want in cases:
        for n_pad in (0, 10_000):
            a = np.concatenate([np.full(n_pad, -np.inf, np.float32), np.array(xs, np.float32)])
            say(f"max_f32 {xs} pad={n_pad}")
            out = rl.red_max_f32(device_view(a, 1, guard=inf if n_pad == 0 else -inf))
            torch.cuda.synchronize()
            assert out.item() == want == float(oracle.max_f32(a)), (xs, out.item())
    say("max_f32 n=0")
    out = rl.red_max_f32(torch.empty(0, device=DEV))
    torch.cuda.synchronize()
    assert out.item() == -inf


def test_max_f32_all_policies():
    a = W.make("normal", (1 << 21) + 1, 78)
    a[(1 << 21) - 77] = 99.0
    x = device_view(a, 3, guard=float("inf"))
    for p in all_flat_policies(bpcs=(2,)):
        say(f"max_f32 policy {p}")
        out = rl.red_max_f32(x, policy=p)
        torch.cuda.synchronize()
        assert out.item() == 99.0, p


def test_sum_i32_all_policies():
    rng = np.random.default_rng(79)
    a = rng.integers(-(2 ** 31), 2 ** 31, (1 << 21) + 5, dtype=np.int64).astype(np.int32)
    want = oracle.sum_i32_i64(a)
    x = device_view(a, 1)
    for p in all_flat_policies(bpcs=(1,)):
        say(f"sum_i32 policy {p}")
        out = rl.red_sum_i32_i64(x, policy=p)
        torch.cuda.synchronize()
        assert int(out.item()) == want, p


# ----------------------------------------------------------------- fused sum, max, sum|x|

def assert_fused_ok(got, a):
    s, m, ab = (float(v) for v in got)
    S, A = oracle.sum_f32(a)
    assert oracle.sum_within_tolerance(s, S, A), ("sum", s, S)
    assert oracle.max_equal(m, oracle.max_f32(a)), ("max", m)
    SA, _ = oracle.sum_f32(np.abs(a))
    assert oracle.sum_within_tolerance(ab, SA, SA if math.isfinite(SA) else 0.0), ("abs", ab, SA)
    # Both sums accumulate in float64 and round once.
    if math.isfinite(S):
        assert f64_contract_ok(s, S, A), ("sum, float64 contract", s, S, A)
    if math.isfinite(SA):
        assert f64_contract_ok(ab, SA, SA), ("sum|x|, float64 contract", ab, SA)


@pytest.mark.parametrize("offset", [0, 1, 3])
def test_sum_max_f32_ragged(offset):
    rng = np.random.default_rng(600 + offset)
    for n in RAGGED:
        say(f"sum_max_f32 n={n} offset={offset}")
        a = (rng.standard_normal(n) * 100).astype(np.float32)
        got = rl.red_sum_max_f32(device_view(a, offset)).cpu().numpy()
        assert_fused_ok(got, a)


def test_sum_max_f32_special():
    nan, inf = float("nan"), float("inf")
    cases = [[1.0, nan, -2.0], [inf, -inf, 3.0], [-inf, -5.0], [-3.0, -1.0, -2.0], [nan, nan]]
    for xs in cases:
        for pad in (0, 3000):
            a = np.concatenate([np.zeros(pad, np.float32), np.array(xs, np.float32)])
            say(f"sum_max_f32 special {xs} pad={pad}")
            got = rl.red_sum_max_f32(device_view(a, 1, guard=0.0)).cpu().numpy()
            S, A = oracle.sum_f32(a)
            SA, _ = oracle.sum_f32(np.abs(a))
            assert oracle.sum_within_tolerance(got[0], S, A), (xs, got[0], S)
            assert got[1] == oracle.max_f32(a)
            assert oracle.sum_within_tolerance(got[2], SA, A), (xs, got[2], SA)
    say("sum_max_f32 n=0")
    got = rl.red_sum_max_f32(torch.empty(0, device=DEV)).cpu().numpy()
    assert got[0] == 0.0 and got[1] == -np.inf and got[2] == 0.0


def test_sum_max_f32_all_policies():
    a = W.make("normal", (1 << 21) + 5, 81)
    x = device_view(a, 2)
    for p in all_flat_policies(bpcs=(2,)):
        say(f"sum_max_f32 policy {p}")
        got = rl.red_sum_max_f32(x, policy=p).cpu().numpy()
        assert_fused_ok(got, a)


# ----------------------------------------------------------------- min, argmax, argmin

@pytest.mark.parametrize("offset", [0, 1, 3])
def test_min_argext_ragged(offset):
    rng = np.random.default_rng(700 + offset)
    for n in RAGGED:
        say(f"min/argmax/argmin n={n} offset={offset}")
        a = rng.standard_normal(n).astype(np.float32)
        x = device_view(a, offset)
        mn = rl.red_min_f32(x)
        am = rl.red_argmax_f32(x)
        ai = rl.red_argmin_f32(x)
        torch.cuda.synchronize()
        assert mn.item() == float(oracle.min_f32(a)), n
        assert int(am.item()) == oracle.argmax_f32(a), n
        assert int(ai.item()) == oracle.argmin_f32(a), n


def test_argext_ties_nan_empty():
    nan, inf = float("nan"), float("inf")
    n = (1 << 20) + 5
    cases = []
    a = np.zeros(n, np.float32)
    cases.append(a)                                         # all equal: index 0
    b = np.zeros(n, np.float32)
    b[[7, 5000, 70000, 900001, n - 1]] = 3.0               # equal maxima in many blocks
    b[[9, 6000, 80000, 800001, n - 2]] = -3.0               # equal minima
    cases.append(b)
    c = np.full(n, nan, np.float32)
    c[[12345, 777777]] = [-1.0, 2.0]                        # NaN everywhere else
    cases.append(c)
    d = np.full(n, -inf, np.float32)
    d[0] = nan                                              # all -inf after a NaN: argmax 1
    cases.append(d)
    e = np.array([0.0, -0.0, 0.0, -0.0], np.float32)        # -0 == +0: index 0
    cases.append(e)
    for k, arr in enumerate(cases):
        for offset in (0, 2):
            say(f"argext case {k} offset={offset}")
            x = device_view(arr, offset, guard=float("inf"))
            am, ai = rl.red_argmax_f32(x), rl.red_argmin_f32(x)
            torch.cuda.synchronize()
            assert int(am.item()) == oracle.argmax_f32(arr), (k, offset)
            assert int(ai.item()) == oracle.argmin_f32(arr), (k, offset)
    for arr in (np.full(100, nan, np.float32), np.zeros(0, np.float32)):
        say(f"argext no number n={arr.size}")
        x = device_view(arr, 1) if arr.size else torch.empty(0, device=DEV)
        assert int(rl.red_argmax_f32(x).item()) == -1
        assert int(rl.red_argmin_f32(x).item()) == -1
        assert rl.red_min_f32(x).item() == float("inf")


def test_argext_tile_cases():
    """Cases aimed at the streaming form of argmax/argmin: each thread keeps
    only the best tile value while streaming and re-reads that tile to find
    the first matching element, so ties inside and across tiles, extremes in
    the last lane of a tile, denormal extremes, signaling NaNs beside the
    extreme, and orders that replace the candidate on every tile all have to
    give the oracle's index."""
    rng = np.random.default_rng(4242)
    n = (1 << 22) + 13
    cases = {}
    a = -rng.random(n, dtype=np.float32)
    a[np.sort(rng.choice(n, 64, replace=False))] = 1.0          # 64 tied maxima
    a[np.sort(rng.choice(n, 64, replace=False))] = -2.0         # 64 tied minima
    cases["ties"] = a
    cases["increasing"] = np.arange(n, dtype=np.float32)       # ties in the f32 rounding
    cases["decreasing"] = -np.arange(n, dtype=np.float32)
    d = (rng.random(n, dtype=np.float32) * 2.0 ** -130).astype(np.float32)   # denormals
    d[[1_000_003, 3_000_001]] = np.float32(2.0 ** -127)
    d[[2_000_002]] = np.float32(0.0)
    cases["denormal"] = d
    s = rng.standard_normal(n).astype(np.float32)
    s.view(np.uint32)[::3] = 0x7F800001                      # signaling NaN bits
    s[[777_777]] = 50.0
    s[[777_778, 777_776]] = -50.0
    cases["snan"] = s
    z = -rng.random(n, dtype=np.float32) - 1.0
    z[[5_000, 5_001, 4_000_000]] = [-0.0, 0.0, 0.0]             # first zero is -0
    cases["signed_zero"] = z
    e = rng.standard_normal(n).astype(np.float32)
    e[[255, 256 * 64 - 1, n - 1]] = 30.0                         # last lanes, array end
    e[[1023, n - 2]] = -30.0
    cases["lane_edges"] = e
    for name, arr in cases.items():
        for offset in (0, 1):
            say(f"argext tile case {name} offset={offset}")
            x = device_view(arr, offset, guard=float("nan"))
            am, ai = rl.red_argmax_f32(x), rl.red_argmin_f32(x)
            torch.cuda.synchronize()
            assert int(am.item()) == oracle.argmax_f32(arr), (name, offset)
            assert int(ai.item()) == oracle.argmin_f32(arr), (name, offset)


def test_min_argext_all_policies():
    n = (1 << 21) + 7
    a = W.make("normal", n, 83)
    a[[3, 100_003, n - 2]] = 9.0          # tied maxima: head, middle, tail
    a[[1, 200_003, n - 1]] = -9.0         # tied minima
    x = device_view(a, 3, guard=float("nan"))
    for p in all_flat_policies(bpcs=(2,)):
        say(f"argext policy {p}")
        am = rl.red_argmax_f32(x, policy=p)
        ai = rl.red_argmin_f32(x, policy=p)
        mn = rl.red_min_f32(x, policy=p)
        torch.cuda.synchronize()
        assert int(am.item()) == 3 and int(ai.item()) == 1 and mn.item() == -9.0, p


# ----------------------------------------------------------------- bf16 / f16 / f64 sums

def half_contract_ok(got, S, A, n):
    """16-bit sums: each 16-byte load's eight values are added in float32 as a
    balanced tree (three roundings on any path, each within 2^-24 of the
    magnitudes added; bfloat16 values are scaled by 1/8 first, exactly), the
    load totals in float64, then one rounding to float32:
    |got - S| <= 2^-24 |S| + 3 * 2^-24 * A + 1e-12 * A, with a float32
    subnormal step per load for sums that rounding absolutely."""
    return abs(float(got) - S) <= U32 * abs(S) + 3.01 * U32 * A + F64_CHAIN * A + (n / 8 + 1) * 2.0 ** -146


def _half_bits(a32, dtype):
    t = torch.from_numpy(a32).to(dtype)
    return t.view(torch.int16).numpy().view(np.uint16), t


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_sum_half_ragged(dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    fn = rl.red_sum_bf16_f32 if dtype == "bf16" else rl.red_sum_f16_f32
    ofn = oracle.sum_bf16 if dtype == "bf16" else oracle.sum_f16
    rng = np.random.default_rng(800)
    for n in RAGGED + [8, 9, 15, 17, 1023 * 8 + 7]:
        for offset in (0, 1, 3, 7):
            say(f"sum {dtype} n={n} offset={offset}")
            bits, t = _half_bits(rng.standard_normal(n).astype(np.float32) * 10, tdt)
            buf = torch.full((n + offset + 16,), float("nan"), dtype=tdt, device=DEV)
            buf[offset:offset + n] = t.to(DEV)
            got = fn(buf[offset:offset + n])
            torch.cuda.synchronize()
            S, A = ofn(bits)
            assert oracle.sum_within_tolerance(got.item(), S, A), (dtype, n, offset, got.item(), S)
            assert half_contract_ok(got.item(), S, A, n), ("16-bit contract", dtype, n, offset, got.item(), S)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_sum_half_exact_and_policies(dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    fn = rl.red_sum_bf16_f32 if dtype == "bf16" else rl.red_sum_f16_f32
    n = (1 << 22) + 13
    ints = (np.arange(n) % 7).astype(np.float32)         # exact in both formats
    t = torch.from_numpy(ints).to(tdt).to(DEV)
    want = float(sum((i % 7) for i in range(7)) * (n // 7) + sum(range(n % 7)))
    say(f"sum {dtype} mod7 exact")
    assert fn(t).item() == want
    for p in all_flat_policies(bpcs=(1,)):
        if p["nontemporal"] == 0 or p["combine"] == 0:
            continue
        say(f"sum {dtype} policy {p}")
        assert fn(t[1:], policy=p).item() == want - 0.0, p


def test_sum_f16_vector_fold():
    """IEEE half sums add each 16-byte load's eight values in float32 before
    float64: denormal halves, the largest half beside tiny ones in one load,
    cancellation inside a load, and infinities and NaN inside a load."""
    rng = np.random.default_rng(810)
    n = (1 << 20) + 5
    cases = {}
    cases["denormal"] = (rng.integers(1, 1024, n).astype(np.uint16))            # all subnormal halves
    big = np.full(n, 0x0001, np.uint16)                                         # 2^-24 everywhere
    big[::8] = 0x7BFF                                                           # 65504 once per load
    cases["wide_range"] = big
    c = rng.standard_normal(n).astype(np.float16)
    c[1::2] = -c[0::2][: c[1::2].size]                                          # x, -x pairs
    cases["cancel"] = c.view(np.uint16)
    d = rng.standard_normal(n).astype(np.float16).view(np.uint16)
    d[[17, 40_000]] = 0x7C00                                                    # +inf
    cases["inf"] = d.copy()
    d[[18]] = 0xFC00                                                            # and -inf: NaN
    cases["inf_minus_inf"] = d.copy()
    e = rng.standard_normal(n).astype(np.float16).view(np.uint16)
    e[[99_999]] = 0x7E00                                                        # NaN
    cases["nan"] = e
    for name, bits in cases.items():
        for offset in (0, 3):
            say(f"sum f16 case {name} offset={offset}")
            t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.float16)
            buf = torch.zeros(n + offset + 8, dtype=torch.float16, device=DEV)
            buf[offset:offset + n] = t.to(DEV)
            got = rl.red_sum_f16_f32(buf[offset:offset + n]).item()
            S, A = oracle.sum_f16(bits)
            assert oracle.sum_within_tolerance(got, S, A), (name, offset, got, S, A)
            if math.isfinite(S):
                assert half_contract_ok(got, S, A, n), ("16-bit contract", name, offset, got, S, A)


def test_sum_bf16_vector_fold():
    """bfloat16 sums add each load's eight values in float32 after scaling
    them by 1/8: values near the top of the range that cancel (an unscaled
    float32 tree would overflow), such values in one load only, subnormal
    values (the scaling must stay exact), infinities and NaN."""
    rng = np.random.default_rng(820)
    n = (1 << 20) + 3
    cases = {}
    big = np.resize(np.array([0x7F60, 0x7F60, 0xFF60, 0xFF60], np.uint16), n)  # +a +a -a -a, a = 2.97e38
    cases["huge_cancel"] = big                                                  # exact sum: a (the tail)
    one = rng.standard_normal(n).astype(np.float32)
    b = (one.view(np.uint32) >> 16).astype(np.uint16)
    b[[1000, 1001, 1002, 1003]] = [0x7F60, 0x7F60, 0xFF60, 0xFF60]             # overflow in one load only
    cases["one_overflow"] = b.copy()
    b[[5000]] = 0x7F80                                                          # +inf
    cases["inf"] = b.copy()
    b[[6000]] = 0xFF80                                                          # and -inf: NaN
    cases["inf_minus_inf"] = b.copy()
    c = (one.view(np.uint32) >> 16).astype(np.uint16)
    c[[77_777]] = 0x7FC0                                                        # NaN
    cases["nan"] = c
    cases["subnormal"] = rng.integers(1, 128, n).astype(np.uint16)              # all subnormal bfloat16
    for name, bits in cases.items():
        for offset in (0, 5):
            say(f"sum bf16 case {name} offset={offset}")
            t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
            buf = torch.zeros(n + offset + 8, dtype=torch.bfloat16, device=DEV)
            buf[offset:offset + n] = t.to(DEV)
            got = rl.red_sum_bf16_f32(buf[offset:offset + n]).item()
            S, A = oracle.sum_bf16(bits)
            assert oracle.sum_within_tolerance(got, S, A), (name, offset, got, S, A)
            if math.isfinite(S):
                assert half_contract_ok(got, S, A, n), ("16-bit contract", name, offset, got, S, A)
            if name == "subnormal":   # the absolute 1e-6 would hide any error here
                assert abs(got - S) <= 1e-5 * A, (offset, got, S, A)


def test_sum_f64():
    rng = np.random.default_rng(900)
    for n in RAGGED:
        for offset in (0, 1):
            say(f"sum f64 n={n} offset={offset}")
            a = rng.standard_normal(n) * 10.0 ** rng.uniform(-5, 5, n)
            buf = torch.full((n + offset + 4,), float("nan"), dtype=torch.float64, device=DEV)
            buf[offset:offset + n] = torch.from_numpy(a).to(DEV)
            got = rl.red_sum_f64(buf[offset:offset + n]).item()
            S, A = oracle.sum_f64(a)
            assert abs(got - S) <= 1e-12 * A + 1e-300, (n, offset, got, S)
    x = torch.arange(1 << 24, dtype=torch.float64, device=DEV)
    say("sum f64 arange 2^24")
    assert rl.red_sum_f64(x).item() == (1 << 24) * ((1 << 24) - 1) / 2


# ----------------------------------------------------------------- rows

ROW_SHAPES = [(70_001, 1), (33_333, 2), (20_011, 4), (2047, 1), (2048, 1), (1023, 2), (511, 4),
              (5000, 7), (3001, 9), (3000, 10), (2999, 11), (2000, 12), (3003, 13), (3000, 14), (3002, 15),
              (3000, 16), (10_001, 8), (768, 3), (767, 3), (4000, 6), (2000, 17), (1500, 21), (1000, 24),
              (999, 31), (1500, 32), (1400, 26), (1, 1), (3, 5), (7, 1000), (65, 257), (4, 0), (1000, 4099), (13, 1), (9, 63),
              (5, 64), (6, 65), (257, 4096), (2, 100_003), (4097, 3), (333, 1024), (50, 513),
              (1000, 4), (777, 16), (301, 32), (129, 128), (77, 200), (33, 8), (1025, 12), (70, 512),
              (200, 33), (100, 511), (1000, 100), (3000, 2), (1, 3), (2, 2), (5, 6), (1001, 6),
              (1, 2048), (2, 1023), (3, 1025), (300, 7), (9, 510), (20_001, 5), (5, 1021), (40, 700), (3, 1023),
              (1, 5000), (2, 1030), (7, 1031), (1, 16), (17, 16), (100_003, 16), (60_001, 7), (50_000, 6),
              (40_001, 25), (30_007, 12), (700, 1028), (300, 1100), (129, 4100), (257, 2052),
              (5000, 1020), (3000, 1025), (2000, 3001), (500, 300), (301, 276), (257, 148), (100, 372),
              (77, 520), (65, 700), (33, 1000),
              # 513-1023 floats: lanes by the rows a 4096-float tile holds (8, 16 or 32),
              # and four-row tiles of odd widths under 584 floats on 2048 waves
              (301, 600), (257, 550), (129, 660), (97, 670), (203, 740), (99, 850), (77, 775),
              (51, 935), (257, 515),
              # 257-511 floats whose 4096-float tile holds 10-12 rows: 4 lanes per row
              (301, 283), (257, 350), (129, 344), (77, 316),
              # a 4096-float tile whose last pass is at most a quarter full yields
              # to a smaller one (2048- or 1024-float tiles on 2048 waves)
              (301, 173), (200, 120), (150, 304), (333, 55)]
ROW_POLICIES = (None, dict(prefetch=1, short_rows=1), dict(prefetch=1, unroll=1, max_blocks=3, short_rows=1),
                dict(prefetch=1, block=256, unroll=4, max_blocks=2, nontemporal=0, short_rows=1),
                dict(short_rows=1), dict(max_blocks=3), dict(max_blocks=1, nontemporal=0),
                dict(short_rows=2), dict(short_rows=3), dict(short_rows=6, max_blocks=3),
                dict(short_rows=9, nontemporal=0), dict(short_rows=5, max_blocks=1),
                dict(cover=2, short_rows=1), dict(cover=2, unroll=16, max_blocks=3, short_rows=1),
                dict(cover=2, block=256, unroll=2, short_rows=1), dict(cover=1, short_rows=1, max_blocks=5),
                dict(short_rows=11), dict(short_rows=14, unroll=16, max_blocks=3), dict(short_rows=16),
                dict(defer=1), dict(defer=1, short_rows=12, max_blocks=2),
                dict(short_rows=17), dict(short_rows=17, max_blocks=3, nontemporal=0),
                dict(lines=1), dict(lines=1, unroll=16, max_blocks=3), dict(lines=2, unroll=8),
                dict(short_rows=3, lines=1), dict(short_rows=11, lines=1, unroll=8),
                dict(short_rows=17, max_blocks=1), dict(short_rows=17, defer=2),
                dict(short_rows=17, defer=2, max_blocks=3), dict(short_rows=17, defer=1), dict(defer=2),
                dict(short_rows=17, defer=2, max_blocks=5, nontemporal=0),
                dict(xcd=1), dict(xcd=2), dict(xcd=3, max_blocks=48), dict(xcd=2, short_rows=1, max_blocks=17),
                dict(xcd=2, cover=2, short_rows=1, max_blocks=40), dict(xcd=4, prefetch=1, short_rows=1, max_blocks=33),
                dict(xcd=2, short_rows=3, max_blocks=20), dict(max_fold=1), dict(max_fold=2),
                dict(max_fold=2, short_rows=3), dict(max_fold=2, short_rows=12, defer=1))


@pytest.mark.parametrize("rows,cols", ROW_SHAPES)
def test_rows_random(rows, cols):
    rng = np.random.default_rng(rows * 7919 + cols)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    if cols:
        a[np.arange(rows), np.arange(rows) % cols] = 50.0 + np.arange(rows)   # planted max
    S, A = oracle.rows_sum_f32(a)
    M = oracle.rows_max_f32(a)
    for offset in (0, 1):
        for p in ROW_POLICIES:
            say(f"rows {rows}x{cols} offset={offset} policy={p}")
            x = device_view(a, offset)
            guard_out = torch.full((rows + 2,), 777.0, device=DEV)
            out_s = guard_out[1:rows + 1]
            rl.red_rows_sum_f32(x, out=out_s, policy=p)
            torch.cuda.synchronize()
            assert guard_out[0].item() == 777.0 and guard_out[-1].item() == 777.0
            got = out_s.cpu().numpy().astype(np.float64)
            assert sums_ok(got, S, A), (rows, cols, p)
            out_m = rl.red_rows_max_f32(x, policy=p)
            torch.cuda.synchronize()
            assert np.array_equal(out_m.cpu().numpy(), M), (rows, cols, p)


@pytest.mark.parametrize("rows,cols,gap", [(1, 8, 0), (2, 4, 0), (3, 3, 0), (100, 1, 0), (9, 1, 0), (7, 1023, 0),
                                           (5, 1021, 3), (1000, 7, 1), (640, 33, 3), (333, 100, 4), (2, 5, 1),
                                           (1, 1000, 0), (4000, 16, 4), (300, 64, 4), (257, 256, 4), (65, 65, 2),
                                           (2048, 2, 0), (77, 511, 1),
                                           # a last tile of one short row whose elements share the
                                           # matrix's last vector with the tile before (unaligned x)
                                           (1022, 1, 0), (2043, 1, 0), (511, 2, 0), (341, 3, 0), (1023, 1, 1),
                                           # rows at a stride of a multiple of 16 floats: element reads
                                           # start at a different element in each row of a pass
                                           (300, 64, 0), (130, 128, 0), (65, 512, 0), (500, 16, 0),
                                           (3000, 32, 0), (40, 960, 0), (200, 48, 16), (100, 60, 4),
                                           (300, 14, 2), (90, 250, 6), (500, 30, 2), (300, 62, 2)])
def test_rows_staged_any_offset(rows, cols, gap):
    # The LDS-staged kernel at every 16-byte offset of x and with short gaps
    # between rows: each tile's span is loaded through its aligned cover, and
    # the matrix's first and last vectors are read element by element when
    # they reach outside it. NaN fills the gaps and the memory on both sides
    # of the matrix, so any element read from outside a row shows in a
    # result.
    ld = cols + gap
    rng = np.random.default_rng(rows * 31 + cols * 7 + gap)
    full = np.full((rows, ld), np.nan, np.float32)
    full[:, :cols] = rng.standard_normal((rows, cols)).astype(np.float32)
    a = np.ascontiguousarray(full[:, :cols])
    S, A = oracle.rows_sum_f32(a)
    M = oracle.rows_max_f32(a)
    for offset in (0, 1, 2, 3):
        for p in (None, dict(defer=1), dict(short_rows=12), dict(short_rows=4, max_blocks=3),
                  dict(short_rows=9, unroll=16)):
            say(f"rows staged {rows}x{cols} ld={ld} offset={offset} policy={p}")
            x = device_view(full, offset)[:, :cols]
            s = rl.red_rows_sum_f32(x, policy=p)
            m = rl.red_rows_max_f32(x, policy=p)
            torch.cuda.synchronize()
            assert sums_ok(s.cpu().numpy().astype(np.float64), S, A), (offset, p)
            assert np.array_equal(m.cpu().numpy(), M), (offset, p)


@pytest.mark.parametrize("rows,cols,ld", [(3, 5, 7), (10, 1000, 1003), (257, 4096, 4100), (64, 63, 64),
                                          (1, 10, 10), (5, 0, 3), (1000, 129, 1024), (300, 16, 20),
                                          (100, 64, 68), (40, 128, 132), (65, 4, 8), (2000, 1000, 1003),
                                          (1500, 1025, 1028), (1200, 2000, 2001), (3000, 17, 24), (700, 33, 48),
                                          (400, 100, 150), (2500, 7, 16), (1777, 3, 8), (900, 128, 192),
                                          (333, 129, 193), (200, 100, 300), (5000, 2, 3)])
def test_rows_strided(rows, cols, ld):
    # Rows spaced ld apart: the gap holds NaN, which must never enter a result.
    rng = np.random.default_rng(rows + cols + ld)
    full = np.full((rows, ld), np.nan, np.float32)
    full[:, :cols] = rng.standard_normal((rows, cols)).astype(np.float32)
    a = np.ascontiguousarray(full[:, :cols])
    S, A = oracle.rows_sum_f32(a)
    M = oracle.rows_max_f32(a)
    for offset in (0, 1):
        for p in ROW_POLICIES:
            say(f"rows strided {rows}x{cols} ld={ld} offset={offset} policy={p}")
            xf = device_view(full, offset)
            x = xf[:, :cols]
            s = rl.red_rows_sum_f32(x, policy=p)
            m = rl.red_rows_max_f32(x, policy=p)
            torch.cuda.synchronize()
            assert sums_ok(s.cpu().numpy().astype(np.float64), S, A), p
            assert np.array_equal(m.cpu().numpy(), M), p


@pytest.mark.parametrize("rows,cols", [(1, 1_000_003), (2, 3_000_017), (7, 1 << 20), (100, 65537),
                                        (1023, 8192), (3, 70_000)])
def test_rows_split_long_rows(rows, cols):
    # Few long rows take the split path (several blocks per row, partials
    # combined per row in order); forced off it must agree too.
    rng = np.random.default_rng(rows * 31 + cols)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    a[np.arange(rows), (np.arange(rows) * 7919) % cols] = 99.0 + np.arange(rows)
    S, A = oracle.rows_sum_f32(a)
    M = oracle.rows_max_f32(a)
    x = device_view(a, 3)
    for p in (None, dict(split=1), dict(split=2, unroll=4), dict(split=2, unroll=16, nontemporal=0),
              dict(split=1, cover=1), dict(split=1, cover=2, unroll=16), dict(split=1, prefetch=1)):
        say(f"rows split {rows}x{cols} policy={p}")
        s = rl.red_rows_sum_f32(x, policy=p)
        m = rl.red_rows_max_f32(x, policy=p)
        torch.cuda.synchronize()
        assert sums_ok(s.cpu().numpy().astype(np.float64), S, A), p
        assert np.array_equal(m.cpu().numpy(), M), p


COL_SHAPES = [(1, 1, 1), (3, 5, 5), (100, 7, 9), (1000, 64, 64), (257, 256, 260), (4099, 1024, 1024),
              (33, 1000, 1001), (2, 4096, 4096), (0, 8, 8), (70_000, 12, 12), (5, 100_003, 100_003),
              (301, 1028, 1032), (77, 2304, 2304), (1000, 3, 3), (777, 33, 33), (500, 65, 65), (3000, 17, 17),
              (200, 257, 257), (99, 1, 1), (4000, 20, 24), (64, 100, 100),
              (1001, 6, 6), (4001, 10, 10), (37, 2, 2), (20_003, 7, 7), (9, 4097, 4097), (5, 3, 3),
              (1000, 260, 260), (333, 516, 516), (41, 300, 300), (3001, 33, 33), (70, 65, 65), (63, 97, 97),
              (300, 1020, 1020), (129, 2040, 2040), (500, 1000, 1020), (77, 765, 765), (45, 1028, 1028),
              (1203, 255, 255), (31, 510, 514),
              # 16-row views whose default launch leaves too few row phases to
              # group per XCD: 4 rows in flight on 1024 waves
              (3001, 1999, 1999), (1700, 2502, 2502),
              # unfolded rows of more than 8192 columns: 4 rows in flight, 2 KiB of
              # a row per wave, unless the shape it replaces is grouped per XCD
              # and this one would not be
              (9, 12000, 12000), (7, 9000, 9004), (40, 50000, 50000), (3, 100000, 100000),
              # short-wide views: row phases rounded down to at most 1024 blocks,
              # with the prefetch where that leaves at most 640
              (272, 30001, 30001), (20, 524292, 524292), (300, 50257, 50257),
              # unfolded wide rows with few phases of many blocks: rounded down
              # (980 blocks), or to 513 blocks with the prefetch
              (48, 100000, 100000), (16, 262148, 262148),
              # rows not 16-byte aligned: four columns per lane from shifted
              # vectors, with and without a spare group per packed row, the
              # wide form's last block past a width of 252 columns per block
              # (and 508 and 1020 at widths 2 and 4), ld a multiple of 4
              # (with the offset 1 runs), and 64 lanes in a row of 252.
              (300, 252, 253), (300, 253, 255), (300, 250, 251), (1000, 509, 511), (100, 1017, 1019),
              (2000, 16, 17), (3000, 5, 7), (1500, 4096, 4097), (400, 125, 128), (123, 2000, 2001)]
COL_POLICIES = (None, dict(vec=1), dict(unroll=1, target_waves=7), dict(unroll=16, nontemporal=0),
                dict(width=2), dict(width=4, unroll=2), dict(width=4, unroll=16, nontemporal=0, target_waves=7),
                dict(prefetch=1), dict(prefetch=1, unroll=1, target_waves=7), dict(width=4, unroll=2, prefetch=1),
                dict(width=2, unroll=16, prefetch=1, nontemporal=0), dict(fold=1), dict(fold=16),
                dict(fold=3, unroll=1, target_waves=7), dict(fold=8, width=4, unroll=2, prefetch=0),
                dict(fold=32), dict(fold=64, unroll=2), dict(order=1), dict(order=2),
                dict(order=2, unroll=1, target_waves=7, prefetch=1), dict(order=3),
                dict(order=3, width=4, unroll=2, target_waves=7), dict(order=3, fold=16, prefetch=0),
                dict(xcd=1), dict(xcd=2), dict(xcd=2, width=4, unroll=2, target_waves=64),
                dict(xcd=2, order=3, target_waves=64), dict(xcd=2, order=2, width=2, unroll=1, target_waves=100))


@pytest.mark.parametrize("rows,cols,ld", COL_SHAPES)
def test_cols(rows, cols, ld):
    rng = np.random.default_rng(rows * 13 + cols * 7 + ld)
    full = np.full((rows, ld), np.nan, np.float32)
    full[:, :cols] = rng.standard_normal((rows, cols)).astype(np.float32)
    if rows and cols:
        full[(np.arange(cols) * 7919) % rows, np.arange(cols)] = 50.0 + np.arange(cols) % 97
    a = np.ascontiguousarray(full[:, :cols])
    S, A = oracle.cols_sum_f32(a)
    M = oracle.cols_max_f32(a)
    for offset in (0, 1):
        for p in COL_POLICIES:
            say(f"cols {rows}x{cols} ld={ld} offset={offset} policy={p}")
            x = device_view(full, offset)[:, :cols]
            s = rl.red_cols_sum_f32(x, policy=p)
            m = rl.red_cols_max_f32(x, policy=p)
            torch.cuda.synchronize()
            assert sums_ok(s.cpu().numpy().astype(np.float64), S, A), p
            assert np.array_equal(m.cpu().numpy(), M), p


@pytest.mark.parametrize("rows,cols", [(40_001, 257), (33_000, 1000), (32_810, 1025), (32_768, 300),
                                       (40_000, 1026), (32_800, 2049), (32_790, 1020), (32_801, 1028)])
def test_cols_line_views(rows, cols):
    # Widths of at least 256 that are not a multiple of 32, with enough rows
    # for the default to read the matrix through 32-row views (16 at 1026
    # columns), each view row whole 128-byte lines; the rows past the last
    # whole view (1-31 of them here, or none) are added in the second pass.
    # At 1020 and 1028 columns the view pitch is a multiple of 255 or 257
    # floats, so the default sweeps the view rows in rotated order.
    rng = np.random.default_rng(rows + 3 * cols)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    a[(np.arange(cols) * 7919) % rows, np.arange(cols)] = 50.0 + np.arange(cols) % 89
    a[-1, ::5] = 80.0                                      # maxima in the last (tail) row
    S, A = oracle.cols_sum_f32(a)
    M = oracle.cols_max_f32(a)
    x = torch.from_numpy(a).to(DEV)
    for p in (None, dict(fold=1)):
        say(f"cols line views {rows}x{cols} policy={p}")
        s = rl.red_cols_sum_f32(x, policy=p)
        m = rl.red_cols_max_f32(x, policy=p)
        torch.cuda.synchronize()
        assert sums_ok(s.cpu().numpy().astype(np.float64), S, A), p
        assert np.array_equal(m.cpu().numpy(), M), p


@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 5), (100, 7), (7, 3), (1000, 64), (33, 1000), (2, 4096),
                                       (3001, 33), (500, 65), (41, 300), (1000, 1), (999, 2), (5, 1021),
                                       (40_001, 257), (2, 2), (1, 5)])
def test_cols_unaligned_views(rows, cols):
    # A contiguous matrix whose x is 1-3 floats past a 16-byte boundary is
    # read through a view that starts at the next boundary, so view column c'
    # holds real column (c' + rot) mod cols; the elements before the view and
    # after its last whole row are added in the second pass. NaN on both
    # sides of the matrix shows any element read from outside it.
    rng = np.random.default_rng(rows * 5 + cols)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    a[(np.arange(cols) * 7919) % rows, np.arange(cols)] = 40.0 + np.arange(cols) % 83
    a[0, :] = np.where(np.arange(cols) % 3 == 0, 90.0, a[0, :])      # maxima before the view
    a[-1, ::2] = 95.0                                                  # and after it
    S, A = oracle.cols_sum_f32(a)
    M = oracle.cols_max_f32(a)
    for offset in (1, 2, 3):
        for p in (None, dict(fold=16), dict(fold=4, unroll=2), dict(width=4, unroll=2), dict(vec=1)):
            say(f"cols unaligned {rows}x{cols} offset={offset} policy={p}")
            x = device_view(a, offset)
            s = rl.red_cols_sum_f32(x, policy=p)
            m = rl.red_cols_max_f32(x, policy=p)
            torch.cuda.synchronize()
            assert sums_ok(s.cpu().numpy().astype(np.float64), S, A), (offset, p)
            assert np.array_equal(m.cpu().numpy(), M), (offset, p)


def _nonfinite_matrix(rows, cols, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    flat = a.reshape(-1)
    k = max(1, flat.size // 97)
    flat[rng.integers(0, flat.size, k)] = np.nan
    flat[rng.integers(0, flat.size, k)] = np.inf
    flat[rng.integers(0, flat.size, k)] = -np.inf
    if rows > 2 and cols > 0:
        a[1, :] = np.nan        # a row of NaN only: its max is -inf
        a[2, :] = -np.inf
    if rows > 0 and cols > 2:
        a[:, 1] = np.nan        # a column of NaN only
        a[:, 2] = np.inf
    return a


def _check_sums(got, S, A, what):
    for i, (g, s_, a_) in enumerate(zip(got, S, A)):
        assert oracle.sum_within_tolerance(g, s_, a_), (what, i, g, s_)


@pytest.mark.parametrize("rows,cols,ld", [(300, 3, 3), (300, 16, 16), (50, 700, 700), (20, 4096, 4096),
                                          (100, 7, 9), (100, 16, 20), (77, 33, 33), (5, 1021, 1021),
                                          (3000, 17, 17), (2000, 32, 32), (1500, 21, 21), (1200, 19, 19),
                                          (900, 23, 23), (800, 31, 31), (1000, 24, 24), (5000, 7, 7)])
def test_rows_nonfinite(rows, cols, ld):
    """NaN and infinities through every row kernel (LDS-staged, packed with
    16-byte and element units, one wave per row): a sum is NaN or the
    infinity exactly when the oracle's is; a max skips NaN (a NaN-only row
    gives -inf)."""
    a = _nonfinite_matrix(rows, cols, rows * 3 + cols)
    full = np.full((rows, ld), 1e30, np.float32)
    full[:, :cols] = a
    S, A = oracle.rows_sum_f32(a)
    M = oracle.rows_max_f32(a)
    for p in (None, dict(short_rows=1), dict(short_rows=2), dict(short_rows=17, defer=1),
              dict(short_rows=17, defer=2, max_blocks=3)):
        say(f"rows nonfinite {rows}x{cols} ld={ld} policy={p}")
        x = device_view(full, 0)[:, :cols]
        s_ = rl.red_rows_sum_f32(x, policy=p)
        m_ = rl.red_rows_max_f32(x, policy=p)
        torch.cuda.synchronize()
        _check_sums(s_.cpu().numpy().astype(np.float64), S, A, p)
        assert np.array_equal(m_.cpu().numpy(), M), p


def test_cols_signalling_nan():
    # Signalling NaNs (quiet bit clear, either sign) never win a column's max,
    # with the hardware max fold (folded views of fewer than 256 columns and
    # short-wide matrices) and with the compare and select; a column of
    # signalling NaNs only gives -inf.
    snans = np.array([0x7F800001, 0x7FA00000, 0xFF800123, 0x7FBFFFFF], np.uint32)
    for rows, cols in ((4000, 7), (3000, 17), (2000, 100), (600, 260), (40, 50257), (300, 4096)):
        rng = np.random.default_rng(rows * 3 + cols)
        a = rng.standard_normal((rows, cols)).astype(np.float32)
        bits = a.view(np.uint32)
        k = max(1, rows * cols // 50)
        idx = rng.choice(rows * cols, size=k, replace=False)
        bits.reshape(-1)[idx] = snans[np.arange(k) % snans.size]
        bits[:, 3] = snans[np.arange(rows) % snans.size]          # a column of signalling NaNs only
        M = oracle.cols_max_f32(a)
        assert M[3] == -np.inf and not np.isnan(M).any()
        for p in (None, dict(unroll=2, width=4), dict(fold=1)):
            say(f"cols signalling NaN {rows}x{cols} policy={p}")
            m = rl.red_cols_max_f32(torch.from_numpy(a).to(DEV), policy=p)
            torch.cuda.synchronize()
            assert np.array_equal(m.cpu().numpy(), M), (rows, cols, p)


def test_rows_signalling_nan():
    # Signalling NaNs (quiet bit clear, either sign) never win a row's max,
    # whichever way the kernel folds the row (compare-and-select, or a
    # maximum instruction that quiets its inputs first: the narrow kernel at
    # some widths, the LDS-staged kernel below 64 floats or with max_fold 2),
    # and make the sum NaN like any other NaN.
    rng = np.random.default_rng(4242)
    snans = np.array([0x7F800001, 0x7FA00000, 0xFF800123, 0x7FBFFFFF], np.uint32)
    for cols in list(range(1, 34)) + [40, 48, 52, 60, 63, 64, 100, 260]:
        rows = 1500 if cols > 8 else 6000
        a = rng.standard_normal((rows, cols)).astype(np.float32)
        bits = a.view(np.uint32)
        k = max(1, a.size // 50)
        idx = rng.integers(0, a.size, k)
        bits.reshape(-1)[idx] = snans[np.arange(k) % snans.size]
        bits[3, :] = snans[np.arange(cols) % snans.size]          # a row of signalling NaNs only
        a[5, :] = -np.inf
        a[7, cols - 1] = np.inf
        S, A = oracle.rows_sum_f32(a)
        M = oracle.rows_max_f32(a)
        assert M[3] == -np.inf and not np.isnan(M).any()
        x = torch.from_numpy(a).to(DEV)
        for p in (None, dict(short_rows=17, defer=1), dict(short_rows=17, defer=2), dict(short_rows=1),
                  dict(max_fold=1), dict(max_fold=2)):
            say(f"rows signalling NaN {rows}x{cols} policy={p}")
            s_ = rl.red_rows_sum_f32(x, policy=p)
            m_ = rl.red_rows_max_f32(x, policy=p)
            torch.cuda.synchronize()
            _check_sums(s_.cpu().numpy().astype(np.float64), S, A, (cols, p))
            assert np.array_equal(m_.cpu().numpy(), M), (cols, p)


@pytest.mark.parametrize("rows,cols,ld", [(1000, 3, 3), (1000, 64, 64), (999, 7, 9), (97, 1031, 1031),
                                          (4001, 10, 10), (500, 12, 12), (999, 64, 65), (300, 1000, 1003),
                                          (2001, 17, 19)])
def test_cols_nonfinite(rows, cols, ld):
    """NaN and infinities through every column path (four columns per lane,
    folded m-row views, one column per lane, packed narrow matrices, shifted
    vectors; the padding between rows is 1e30, which a shifted load reads
    but no column may take)."""
    a = _nonfinite_matrix(rows, cols, rows * 5 + cols)
    full = np.full((rows, ld), 1e30, np.float32)
    full[:, :cols] = a
    S, A = oracle.cols_sum_f32(a)
    M = oracle.cols_max_f32(a)
    for p in (None, dict(vec=1), dict(target_waves=7, unroll=1)):
        say(f"cols nonfinite {rows}x{cols} ld={ld} policy={p}")
        x = device_view(full, 0)[:, :cols]
        s_ = rl.red_cols_sum_f32(x, policy=p)
        m_ = rl.red_cols_max_f32(x, policy=p)
        torch.cuda.synchronize()
        _check_sums(s_.cpu().numpy().astype(np.float64), S, A, p)
        assert np.array_equal(m_.cpu().numpy(), M), p


def test_cols_mod7_exact():
    rows, cols = 4097, 1031
    say("cols mod7")
    a = W.pattern_rows_mod7(rows, cols)
    S, _ = oracle.cols_sum_f32(a)
    out = rl.red_cols_sum_f32(device_view(a, 0))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), S)


def test_rows_mod7_exact():
    rows, cols = 1031, 4097
    say(f"rows mod7 {rows}x{cols}")
    a = W.pattern_rows_mod7(rows, cols)
    x = device_view(a, 2)
    S, _ = oracle.rows_sum_f32(a)
    out = rl.red_rows_sum_f32(x)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), S)


def test_rows_zero_rows():
    say("rows 0x5")
    out = rl.red_rows_sum_f32(torch.empty((0, 5), device=DEV))
    assert out.numel() == 0


def test_rows_policies():
    a = W.make("uniform01", 300 * 1027, 9).reshape(300, 1027)
    S, A = oracle.rows_sum_f32(a)
    M = oracle.rows_max_f32(a)
    x = device_view(a, 1)
    for block in (64, 128, 256, 512):
        for unroll in (1, 2, 4, 8, 16):
            for nt, pf in ((0, 0), (1, 0), (0, 1), (1, 1)):
                for mb in (1, 7, 1 << 20):
                    say(f"rows policy block={block} unroll={unroll} nt={nt} pf={pf} max_blocks={mb}")
                    p = dict(block=block, unroll=unroll, nontemporal=nt, max_blocks=mb, prefetch=pf)
                    s = rl.red_rows_sum_f32(x, policy=p)
                    m = rl.red_rows_max_f32(x, policy=p)
                    torch.cuda.synchronize()
                    assert sums_ok(s.cpu().numpy(), S, A)
                    assert np.array_equal(m.cpu().numpy(), M)


# ----------------------------------------------------------------- ablation

def _block_sums_mod7(n, span):
    idx = np.arange(n, dtype=np.int64) % 7
    nb = (n + span - 1) // span
    pad = np.zeros(nb * span, np.int64)
    pad[:n] = idx
    return pad.reshape(nb, span).sum(axis=1).astype(np.float32)


@pytest.mark.parametrize("rung", [1, 2, 3, 4, 5, 6])
def test_ablation_rungs(rung):
    for row in __import__("oracle_pins").read_golden("lesson_demo3_mod7.txt"):
        n, want = int(row["n"]), int(row["expected"])
        say(f"rung {rung} mod7 n={n}")
        out, partials = rl.red_ablate_sum_f32(rung, device_view(W.pattern_mod7(n)))
        torch.cuda.synchronize()
        assert out.item() == want
        if rung <= 5:
            span = 512 if rung >= 4 else 256
            assert np.array_equal(partials.cpu().numpy(), _block_sums_mod7(n, span))
    for n in (1, 255, 257, 1000, (1 << 20) + 3):
        say(f"rung {rung} random n={n}")
        a = W.make("normal", n, 400 + n % 97)
        out, _ = rl.red_ablate_sum_f32(rung, device_view(a, 1))
        torch.cuda.synchronize()
        if rung == 6:
            assert_sum_ok(out.item(), a)
        else:
            # Rungs 1-5 are the lesson's versions: float32 block trees (at most
            # 9 additions deep), so only the 1e-5 acceptance bound applies.
            S, A = oracle.sum_f32(a)
            assert oracle.sum_within_tolerance(out.item(), S, A), (rung, n, out.item(), S)


def test_ablation_partials_only():
    n = (1 << 20) + 3
    a = W.pattern_mod7(n)
    x = device_view(a, 1)
    for rung in range(1, 6):
        say(f"rung {rung} partials only n={n}")
        out, partials = rl.red_ablate_sum_f32(rung, x, partials_only=True)
        torch.cuda.synchronize()
        assert out is None
        span = 512 if rung >= 4 else 256
        assert np.array_equal(partials.cpu().numpy(), _block_sums_mod7(n, span))


# ----------------------------------------------------------------- probes

def test_wave_reduce_primitive_matches_lane_model():
    # The DPP wave reduce against the lane-by-lane CPU model of the same
    # pairing: bit-exact for float64 sums, exact for int64 sums and max.
    from lane_models import add, dpp_reduce, max_rule
    rng = np.random.default_rng(21)
    waves = 64
    f = (rng.standard_normal(waves * 64) * 10.0 ** rng.uniform(-6, 6, waves * 64)).astype(np.float64)
    f[:64] = [1e16 if i % 16 == 0 else 1.0 for i in range(64)]      # order-sensitive wave
    say("wave reduce f64")
    got = rl.red_probe_wave_reduce("sum_f64", torch.from_numpy(f).to(DEV)).cpu().numpy()
    want = [dpp_reduce(f[64 * w:64 * (w + 1)].tolist(), add, 0.0) for w in range(waves)]
    assert got.tolist() == want
    i = rng.integers(-(2 ** 62), 2 ** 62, waves * 64, dtype=np.int64)
    say("wave reduce i64")
    got = rl.red_probe_wave_reduce("sum_i64", torch.from_numpy(i).to(DEV)).cpu().numpy()
    want = [(sum(i[64 * w:64 * (w + 1)].tolist()) + 2 ** 63) % 2 ** 64 - 2 ** 63 for w in range(waves)]
    assert got.tolist() == want
    m = rng.standard_normal(waves * 64).astype(np.float32)
    m[5] = np.nan
    say("wave reduce max")
    got = rl.red_probe_wave_reduce("max_f32", torch.from_numpy(m).to(DEV)).cpu().numpy()
    want = [dpp_reduce(m[64 * w:64 * (w + 1)].tolist(), max_rule, -math.inf) for w in range(waves)]
    assert got.tolist() == [np.float32(v) for v in want]


def test_shfl_down_primitive_matches_lane_model():
    from lane_models import shfl_down
    v = np.arange(64, dtype=np.float32) * 1.5 - 7
    x = torch.from_numpy(v).to(DEV)
    for off in (0, 1, 2, 4, 8, 16, 31, 32, 33, 63, 64):
        say(f"shfl_down offset={off}")
        got = rl.red_probe_shfl_down_f32(x, off).cpu().numpy()
        assert got.tolist() == shfl_down(v.tolist(), off), off


def test_graph_replay_matches_eager():
    # Captured calls (after a first eager call per stream, so the workspace
    # and the column scratch exist) replay correctly several times with eager
    # work in between.
    a = W.make("normal", (1 << 22) + 3, 31)
    r = W.make("uniform01", 300 * 1001, 32).reshape(300, 1001)
    x, xr = device_view(a, 1), device_view(r, 2)
    xh = torch.from_numpy(a).to(DEV).to(torch.float16)
    outs = [torch.empty((), device=DEV), torch.empty((), device=DEV), torch.empty(300, device=DEV),
            torch.empty((), dtype=torch.int64, device=DEV), torch.empty((), device=DEV),
            torch.empty(3, device=DEV), torch.empty(1001, device=DEV)]

    def calls():
        rl.red_sum_f32(x, out=outs[0])
        rl.red_max_f32(x, out=outs[1])
        rl.red_rows_sum_f32(xr, out=outs[2])
        rl.red_argmax_f32(x, out=outs[3])
        rl.red_sum_f16_f32(xh, out=outs[4])
        rl.red_sum_max_f32(x, out=outs[5])
        rl.red_cols_sum_f32(xr, out=outs[6])

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        calls()
        torch.cuda.synchronize()
        eager = [o.clone() for o in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            calls()
    torch.cuda.synchronize()
    for k in range(4):
        say(f"graph replay {k}")
        for o in outs:
            o.zero_()
        rl.red_sum_f32(x)                      # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e)


def test_graph_survives_scratch_growth():
    # A graph holds the column scratch pointer it was captured with; a later
    # eager call on the same stream that needs more scratch must not free it,
    # so the graph replays correctly afterwards.
    small = device_view(W.make("normal", 64 * 256, 44).reshape(64, 256), 0)
    big = device_view(W.make("normal", 4096 * 1024, 45).reshape(4096, 1024), 0)
    out = torch.empty(256, device=DEV)
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    say("graph over column scratch, then scratch growth")
    with torch.cuda.stream(cs):
        want = rl.red_cols_sum_f32(small).clone()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            rl.red_cols_sum_f32(small, out=out)
        big_sum = rl.red_cols_sum_f32(big, policy=dict(target_waves=4096, unroll=1))  # grows the scratch
    torch.cuda.synchronize()
    S, A = oracle.cols_sum_f32(big.cpu().numpy())
    assert sums_ok(big_sum.cpu().numpy().astype(np.float64), S, A)
    for k in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), k


def test_capture_without_workspace_is_refused():
    # A fresh stream has no workspace yet: a call captured on it must fail
    # with RED_ERR_CAPTURE before touching the stream, leaving the capture
    # usable; after one eager call the same capture works.
    x = device_view(W.make("normal", 1 << 16, 41), 0)
    out = torch.empty((), device=DEV)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    say("capture on a fresh stream")
    with torch.cuda.stream(cap):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            with pytest.raises(rl.RedError) as ei:
                rl.red_sum_f32(x, out=out)
            out.fill_(1.0)
        assert ei.value.status == rl.RED_ERR_CAPTURE
    torch.cuda.synchronize()
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert out.item() == 1.0
    say("capture after an eager call")
    with torch.cuda.stream(cap):
        want = rl.red_sum_f32(x).item()
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=cap):
            rl.red_sum_f32(x, out=out)
    torch.cuda.synchronize()
    out.zero_()
    g2.replay()
    torch.cuda.synchronize()
    assert out.item() == want
    say("column call needing more scratch under capture")
    small = device_view(W.make("normal", 64 * 256, 42).reshape(64, 256), 0)
    big = device_view(W.make("normal", 4096 * 1024, 43).reshape(4096, 1024), 0)
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        rl.red_cols_sum_f32(small)                 # scratch sized for the small shape
        torch.cuda.synchronize()
        g3 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g3, stream=cs):
            with pytest.raises(rl.RedError) as ei:
                rl.red_cols_sum_f32(big, policy=dict(target_waves=4096, unroll=1))
        assert ei.value.status == rl.RED_ERR_CAPTURE
    torch.cuda.synchronize()


def test_lds_stride_probe():
    words = 64 * 65
    for stride in (1, 2, 32, 33, 0, -1, 4095):
        for iters in (0, 1, 77):
            say(f"lds probe stride={stride} iters={iters}")
            sink = torch.zeros(1, dtype=torch.int32, device=DEV)
            rl.red_probe_lds_stride(stride, iters, sink)
            torch.cuda.synchronize()
            base = [l // 2 if stride < 0 else (l * stride) % words for l in range(64)]
            want = (iters * sum(base)) % (1 << 32)
            assert int(sink.item()) & 0xFFFFFFFF == want, (stride, iters)



def test_probes():
    n = (1 << 20) + 3
    say("probe copy/read")
    a = W.make("normal", n, 12)
    x = torch.from_numpy(a).to(DEV)
    y = torch.empty_like(x)
    rl.red_probe_copy_f32(x, y)
    sink = rl.red_probe_read_f32(x[1:])
    torch.cuda.synchronize()
    assert torch.equal(x, y)
    want = int(np.bitwise_xor.reduce(a[1:].view(np.uint32)))
    assert int(sink.item()) & 0xFFFFFFFF == want
    cu, arch = rl.red_device_info()
    assert cu > 0 and arch.startswith("gfx950")


# ----------------------------------------------------------------- full sizes
# The five workloads at their real sizes, with the default launch shapes
# (the ones the benchmark times).

def _load(name):
    say(f"generate {name}")
    a = W.workload(name)
    say(f"upload {name}")
    x = torch.from_numpy(a).to(DEV)
    torch.cuda.synchronize()
    return a, x


def test_full_sum_f32_2p20():
    a, x = _load("sum_f32_2p20")
    say("red_sum_f32 sum_f32_2p20")
    assert_sum_ok(gpu_sum(x), a)


def test_full_sum_i32_2p24():
    a, x = _load("sum_i32_2p24")
    say("red_sum_i32_i64 sum_i32_2p24")
    out = rl.red_sum_i32_i64(x)
    torch.cuda.synchronize()
    assert int(out.item()) == oracle.sum_i32_i64(a)


def test_full_sum_max_f32_2p28():
    a, x = _load("sum_max_f32_2p28")
    say("red_sum_f32 sum_max_f32_2p28")
    got = gpu_sum(x)
    assert_sum_ok(got, a)
    assert gpu_sum(x) == got
    say("red_max_f32 sum_max_f32_2p28")
    m = rl.red_max_f32(x)
    torch.cuda.synchronize()
    assert m.item() == float(oracle.max_f32(a))
    del x
    torch.cuda.empty_cache()


def test_full_sum_i32_bits_2p28():
    # The int32 sum at the 1 GiB size the bench times: the 2^28 words of the
    # normal array read as int32 (large values of both signs), bit-exact
    # against the oracle's int64 sum.
    a, x = _load("sum_max_f32_2p28")
    say("red_sum_i32_i64 over the bits of sum_max_f32_2p28")
    out = rl.red_sum_i32_i64(x.view(torch.int32))
    torch.cuda.synchronize()
    assert int(out.item()) == oracle.sum_i32_i64(a.view(np.int32))
    del x
    torch.cuda.empty_cache()


def test_full_sum_max_f32_fused_2p28():
    a, x = _load("sum_max_f32_2p28")
    say("red_sum_max_f32 sum_max_f32_2p28")
    got = rl.red_sum_max_f32(x).cpu().numpy()
    assert_fused_ok(got, a)
    del x
    torch.cuda.empty_cache()


def test_full_min_argmax_2p28():
    a, x = _load("sum_max_f32_2p28")
    say("red_min_f32 / red_argmax_f32 / red_argmin_f32 sum_max_f32_2p28")
    mn, am, ai = rl.red_min_f32(x), rl.red_argmax_f32(x), rl.red_argmin_f32(x)
    torch.cuda.synchronize()
    assert mn.item() == float(oracle.min_f32(a))
    assert int(am.item()) == oracle.argmax_f32(a)
    assert int(ai.item()) == oracle.argmin_f32(a)
    del x
    torch.cuda.empty_cache()


def test_full_sparse_ones_2p28():
    n = 1 << 28
    say("sum_f32 sparse ones (every 32nd) n=2^28")
    x = torch.zeros(n, device=DEV)
    x[::32] = 1.0
    assert gpu_sum(x) == float(n // 32)
    del x
    torch.cuda.empty_cache()


def test_full_rows_65536x4096():
    a, x = _load("rows_f32_65536x4096")
    say("red_rows_sum_f32 / red_rows_max_f32 rows_f32_65536x4096")
    s = rl.red_rows_sum_f32(x)
    m = rl.red_rows_max_f32(x)
    torch.cuda.synchronize()
    S, A = oracle.rows_sum_f32(a)
    assert sums_ok(s.cpu().numpy().astype(np.float64), S, A)
    assert np.array_equal(m.cpu().numpy(), oracle.rows_max_f32(a))
    del x
    torch.cuda.empty_cache()


def test_full_rows_short_1gib():
    # The 1 GiB rows workload viewed as (2^28 // cols) x cols rows, the shapes
    # the widths benchmark times. Every row of every view is compared with
    # the oracle. By default the LDS-staged kernel holds each wave's row
    # results until its last tile, and the narrow kernel (from 6 floats)
    # holds them for a burst of tiles; defer=1 stores them tile by tile. Each
    # row is reduced the same way in both, so the floats must also be
    # identical.
    a, x = _load("rows_f32_65536x4096")
    flat = a.reshape(-1)
    for cols in (1, 3, 4, 7, 12, 16, 17, 21, 32, 64, 100, 120, 173, 256, 283, 378, 515, 600, 700, 850, 1000, 1025,
                 3001):
        rows = flat.size // cols
        say(f"red_rows_sum_f32 / red_rows_max_f32 rows_f32_65536x4096 as {rows}x{cols}, held and tile by tile")
        v = x.view(-1)[: rows * cols].view(rows, cols)
        s0, m0 = rl.red_rows_sum_f32(v), rl.red_rows_max_f32(v)
        s1, m1 = rl.red_rows_sum_f32(v, policy=dict(defer=1)), rl.red_rows_max_f32(v, policy=dict(defer=1))
        torch.cuda.synchronize()
        assert torch.equal(s0, s1) and torch.equal(m0, m1), cols
        mat = flat[: rows * cols].reshape(rows, cols)
        say(f"oracle rows {rows}x{cols}")
        S, A = oracle.rows_sum_f32(mat)
        assert sums_ok(s0.cpu().numpy(), S, A), cols
        assert np.array_equal(m0.cpu().numpy(), oracle.rows_max_f32(mat)), cols
    del x
    torch.cuda.empty_cache()


def test_full_cols_65536x4096():
    a, x = _load("rows_f32_65536x4096")
    say("red_cols_sum_f32 / red_cols_max_f32 rows_f32_65536x4096")
    s = rl.red_cols_sum_f32(x)
    m = rl.red_cols_max_f32(x)
    torch.cuda.synchronize()
    S, A = oracle.cols_sum_f32(a)
    assert sums_ok(s.cpu().numpy().astype(np.float64), S, A)
    assert np.array_equal(m.cpu().numpy(), oracle.cols_max_f32(a))
    del x
    torch.cuda.empty_cache()


def test_full_cols_strided_1gib():
    # The 1 GiB rows workload viewed as rows of ld floats of which the first
    # cols are the matrix, the strided shapes the column-stride benchmark
    # times (default launch shapes: shifted vectors where rows do not start
    # 16-byte aligned, XCD-grouped blocks where the pitch is not a power of
    # two). Every column is compared with the oracle.
    a, x = _load("rows_f32_65536x4096")
    flat = a.reshape(-1)
    for cols, ld in ((4096, 4097), (4096, 4100), (1020, 1021), (256, 257), (64, 65), (17, 19), (5, 7)):
        rows = flat.size // ld
        say(f"red_cols_sum_f32 / red_cols_max_f32 rows_f32_65536x4096 as {rows}x{cols}, ld {ld}")
        v = x.view(-1)[: rows * ld].view(rows, ld)[:, :cols]
        s = rl.red_cols_sum_f32(v)
        m = rl.red_cols_max_f32(v)
        torch.cuda.synchronize()
        mat = np.ascontiguousarray(flat[: rows * ld].reshape(rows, ld)[:, :cols])
        say(f"oracle cols {rows}x{cols}")
        S, A = oracle.cols_sum_f32(mat)
        assert sums_ok(s.cpu().numpy().astype(np.float64), S, A), (cols, ld)
        assert np.array_equal(m.cpu().numpy(), oracle.cols_max_f32(mat)), (cols, ld)
        del mat
    del x
    torch.cuda.empty_cache()


def test_full_cols_folded_1gib():
    # The 1 GiB rows workload viewed as contiguous (2^28 // cols) x cols
    # matrices that the column kernels read through 32- or 16-row views.
    # Views of at most 224 blocks of 256 columns whose default launch has too
    # few row phases to group per XCD (300, 1000 and 1025 columns in 32-row
    # views, 2502 in 16-row views) take 4 rows in flight on 1024 waves; 2500
    # and 3000 columns keep the default. Unfolded rows of more than 8192
    # columns (12000, 100000) take 4 rows in flight with 2 KiB of a row per
    # wave; 50000 keeps the short-wide shape, whose blocks are grouped per
    # XCD. Every column is compared with the oracle.
    a, x = _load("rows_f32_65536x4096")
    flat = a.reshape(-1)
    for cols in (300, 1000, 1025, 2500, 2502, 3000, 12000, 50000, 100000):
        rows = flat.size // cols
        say(f"red_cols_sum_f32 / red_cols_max_f32 rows_f32_65536x4096 as {rows}x{cols}")
        v = x.view(-1)[: rows * cols].view(rows, cols)
        s = rl.red_cols_sum_f32(v)
        m = rl.red_cols_max_f32(v)
        torch.cuda.synchronize()
        mat = flat[: rows * cols].reshape(rows, cols)
        say(f"oracle cols {rows}x{cols}")
        S, A = oracle.cols_sum_f32(mat)
        assert sums_ok(s.cpu().numpy().astype(np.float64), S, A), cols
        assert np.array_equal(m.cpu().numpy(), oracle.cols_max_f32(mat)), cols
    del x
    torch.cuda.empty_cache()


def test_full_sum_f32_1e9p7():
    a, x = _load("sum_f32_1e9p7")
    say("red_sum_f32 sum_f32_1e9p7")
    got = gpu_sum(x)
    say("oracle sum_f32_1e9p7")
    assert_sum_ok(got, a)
    say("red_sum_f32 sum_f32_1e9p7 offset view")
    assert_sum_ok(gpu_sum(x[1:]), a[1:])
    del x
    torch.cuda.empty_cache()


def test_full_sparse_ones_1e9p7():
    n = 1_000_000_007
    say("sum_f32 sparse ones (every 64th) n=1e9+7")
    x = torch.zeros(n, device=DEV)
    x[::64] = 1.0
    assert gpu_sum(x) == float(len(range(0, n, 64)))
    assert gpu_sum(x[3:]) == float(len(range(64, n, 64)))
    del x
    torch.cuda.empty_cache()


def test_beyond_2p32_elements():
    """More than 2^32 elements (16 GiB of float32), so every element index and
    count needs 64 bits: sparse ones with one planted maximum past index 2^32,
    read as float32, as int32 bit patterns, as a 65536 x 65536 matrix by rows
    and by columns, as two rows of 2^31 (the split-row path), by columns at
    an odd leading dimension, and as rows of 1025 floats from x and x + 1."""
    n = (1 << 32) + 7
    p = (1 << 32) + 3                       # past 2^32, not a multiple of 64
    say(f"n = 2^32 + 7 ({4 * n / 2**30:.1f} GiB)")
    x = torch.zeros(n, device=DEV)
    x[::64] = 1.0
    x[p] = 5.0
    ones = (n + 63) // 64
    torch.cuda.synchronize()
    say("sum / max / min / argmax / argmin beyond 2^32")
    assert gpu_sum(x) == float(np.float32(ones + 5))
    assert gpu_sum(x[1:]) == float(np.float32(ones - 1 + 5))
    assert rl.red_max_f32(x).item() == 5.0
    assert rl.red_min_f32(x).item() == 0.0
    assert int(rl.red_argmax_f32(x).item()) == p
    assert int(rl.red_argmin_f32(x).item()) == 1
    assert int(rl.red_argmax_f32(x[5:]).item()) == p - 5
    fused = rl.red_sum_max_f32(x).cpu().numpy()
    assert fused[0] == np.float32(ones + 5) and fused[1] == 5.0 and fused[2] == np.float32(ones + 5)
    say("int32 bit patterns beyond 2^32")
    want = ones * 0x3F800000 + 0x40A00000            # bits of 1.0f and 5.0f
    assert int(rl.red_sum_i32_i64(x.view(torch.int32)).item()) == want
    say("rows and columns of a 65536 x 65536 view")
    m = x[: 1 << 32].view(1 << 16, 1 << 16)
    assert torch.all(rl.red_rows_sum_f32(m) == 1024.0)
    assert torch.all(rl.red_rows_max_f32(m) == 1.0)
    c = rl.red_cols_sum_f32(m)
    want_c = torch.zeros(1 << 16, device=DEV)
    want_c[::64] = float(1 << 16)
    assert torch.equal(c, want_c)
    assert torch.equal(rl.red_cols_max_f32(m), (want_c > 0).float())
    say("two rows of 2^31 (split rows)")
    r2 = x[: 1 << 32].view(2, 1 << 31)
    assert torch.all(rl.red_rows_sum_f32(r2) == float(1 << 25))
    # Columns at an odd leading dimension (shifted vectors, blocks grouped
    # per XCD): 65535 rows of 65537 floats span 2^32 - 1 elements. Element
    # r * 65537 + c is a one when r + c is a multiple of 64 (65537 = 1 mod 64).
    ld = 65537
    rows_s = n // ld
    say(f"columns of a {rows_s} x 65536 view at ld {ld}")
    ms = x[: rows_s * ld].view(rows_s, ld)[:, : 1 << 16]
    r0 = (-np.arange(1 << 16)) % 64
    want_s = np.where(r0 < rows_s, (rows_s - 1 - r0) // 64 + 1, 0).astype(np.float32)
    assert np.array_equal(rl.red_cols_sum_f32(ms).cpu().numpy(), want_s)
    assert np.array_equal(rl.red_cols_max_f32(ms).cpu().numpy(), (want_s > 0).astype(np.float32))
    # Rows of 1025 floats (the cover kernel, blocks dealt to the XCDs in
    # runs): 4190212 rows span more than 2^32 elements; the planted 5.0 sits
    # in the last row.
    rows_r = n // 1025
    say(f"rows of a {rows_r} x 1025 view")
    mr = x[: rows_r * 1025].view(rows_r, 1025)
    lo = np.arange(rows_r, dtype=np.int64) * 1025
    want_r = ((lo + 1024) // 64 - (lo + 63) // 64 + 1).astype(np.float64)
    last = p // 1025
    want_r[last] += 5.0
    want_m = np.where(want_r > 0, 1.0, 0.0).astype(np.float32)
    want_m[last] = 5.0
    assert np.array_equal(rl.red_rows_sum_f32(mr).cpu().numpy(), want_r.astype(np.float32))
    assert np.array_equal(rl.red_rows_max_f32(mr).cpu().numpy(), want_m)
    # The same rows from x + 1 (rows that do not start 16-byte aligned).
    mr1 = x[1: 1 + rows_r * 1025].view(rows_r, 1025)
    lo1 = lo + 1
    want_r1 = ((lo1 + 1024) // 64 - (lo1 + 63) // 64 + 1).astype(np.float64)
    if (p - 1) // 1025 < rows_r:
        want_r1[(p - 1) // 1025] += 5.0
    assert np.array_equal(rl.red_rows_sum_f32(mr1).cpu().numpy(), want_r1.astype(np.float32))
    del x, m, r2, ms, mr, mr1
    torch.cuda.empty_cache()


def test_concurrent_streams_from_host_threads():
    # Calls from several host threads, each on its own stream, run at once
    # (ctypes releases the interpreter lock during each call): every stream
    # gets its own workspace and scratch, created under the library's lock,
    # and every result equals the one computed alone.
    import threading
    arrays = [device_view(W.make("normal", (1 << 20) + 7 * k, 60 + k), k % 4) for k in range(4)]
    mats = [device_view(W.make("uniform01", 700 * (300 + k), 70 + k).reshape(700, 300 + k), 0) for k in range(4)]
    want = []
    for a, m in zip(arrays, mats):
        want.append((rl.red_sum_f32(a).clone(), rl.red_max_f32(a).clone(), rl.red_rows_sum_f32(m).clone(),
                     rl.red_cols_sum_f32(m).clone(), rl.red_argmax_f32(a).clone()))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [None] * 4
    errors = []

    def work(k):
        try:
            with torch.cuda.stream(streams[k]):
                res = None
                for _ in range(20):
                    res = (rl.red_sum_f32(arrays[k]), rl.red_max_f32(arrays[k]), rl.red_rows_sum_f32(mats[k]),
                           rl.red_cols_sum_f32(mats[k]), rl.red_argmax_f32(arrays[k]))
                streams[k].synchronize()
                got[k] = res
        except Exception as e:  # reported below, in the test's thread
            errors.append(e)

    say("four host threads, four streams")
    threads = [threading.Thread(target=work, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(4):
        for g, w in zip(got[k], want[k]):
            assert torch.equal(g, w), k
