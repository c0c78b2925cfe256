"""The seeded input generators: determinism, shapes, dtypes and ranges."""
import numpy as np

import workloads as W


def test_named_workloads_listed():
    assert set(W.WORKLOADS) == {"sum_f32_2p20", "sum_i32_2p24", "sum_max_f32_2p28",
                                "rows_f32_65536x4096", "sum_f32_1e9p7"}
    for name in W.WORKLOADS:
        d = W.describe(name)
        assert d["chunk"] == 1 << 24


def test_make_is_deterministic_and_chunked():
    a = W.make("normal", (1 << 24) + 1000, 2)
    b = W.make("normal", (1 << 24) + 1000, 2)
    assert np.array_equal(a, b)
    c = W.make("normal", 1 << 24, 2)
    assert np.array_equal(a[: 1 << 24], c)
    assert not np.array_equal(W.make("normal", 1000, 3), W.make("normal", 1000, 2))


def test_small_workload_values():
    x = W.workload("sum_f32_2p20")
    assert x.dtype == np.float32 and x.shape == (1 << 20,)
    assert x.min() >= -1.0 and x.max() <= 1.0
    y = W.make("int_pm1000", 100_000, 1)
    assert y.dtype == np.int32 and y.min() == -1000 and y.max() == 1000
    m = W.make("mixture", 1_000_000, 4)
    wide = np.abs(m) > 1.0
    assert 0.008 < wide.mean() < 0.012          # about 1% wide component
    assert np.abs(m).max() <= 1e4
    u = W.make("uniform01", 100_000, 3)
    assert u.min() >= 0.0 and u.max() < 1.0


def test_patterns():
    assert np.array_equal(W.pattern_mod7(10), np.float32([0, 1, 2, 3, 4, 5, 6, 0, 1, 2]))
    e = W.pattern_every(130, 64)
    assert e.sum() == 3 and e[0] == 1 and e[64] == 1 and e[128] == 1
    t = W.pattern_tags(100, [0, 99, 50])
    assert t[0] == 1 and t[99] == 2 and t[50] == 4 and t.sum() == 7
    r = W.pattern_rows_mod7(3, 9)
    assert r[2, 5] == 0 and r[1, 0] == 1
