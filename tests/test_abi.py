"""The C ABI without a GPU: exported symbols, status strings, argument checks.

Argument errors must be reported as RED_ERR_INVALID_ARG before any HIP call;
on a machine without a GPU any HIP call would turn the status into
RED_ERR_NO_DEVICE, so these checks also show the order. No call here
reaches a kernel.
"""
import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import reduction_libred_amd as rl  # noqa: E402

INVALID, NO_DEVICE = rl.RED_ERR_INVALID_ARG, rl.RED_ERR_NO_DEVICE


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(red_[a-z0-9_]+)\s*\(", text))
    return names


def exported_symbols():
    out = subprocess.run(["nm", "-D", "--defined-only", rl.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.split()[-2:-1] == ["T"]}


def test_exports_match_headers():
    rl.lib()
    decl = declared_symbols()
    assert len(decl) >= 21
    assert decl == exported_symbols()
    assert decl == set(rl.SIGNATURES)
    for name in decl:
        assert getattr(rl.lib(), name) is not None


def test_status_strings_and_version():
    L = rl.lib()
    for code in range(7):
        assert L.red_status_string(code) != b"unknown red_status", code
    assert L.red_status_string(99) == b"unknown red_status"
    assert rl.red_version().startswith("libred")


def _p(v):
    return ctypes.c_void_p(v)


A, B = 0x10000, 0x20000            # aligned fake addresses, never dereferenced


def test_flat_argument_errors():
    L = rl.lib()
    for f in (L.red_sum_f32, L.red_sum_f32_noalloc, L.red_max_f32, L.red_sum_i32_i64):
        assert f(None, 4, _p(B), None) == INVALID                 # null x, n > 0
        assert f(_p(A), 4, None, None) == INVALID                 # null out
        assert f(_p(A + 1), 4, _p(B), None) == INVALID            # misaligned x
        assert f(_p(A), 4, _p(B + 2), None) == INVALID            # misaligned out
        assert f(_p(A), 4, _p(A + 8), None) == INVALID            # out inside x
        assert f(_p(A), rl.RED_MAX_N + 1, _p(B), None) == INVALID
    assert L.red_sum_i32_i64(_p(A), 4, _p(B + 4), None) == INVALID  # int64 out needs 8
    bad = rl.FlatPolicy(100, 8, 4, 1)
    assert L.red_sum_f32_with(_p(A), 4, _p(B), ctypes.byref(bad), None) == INVALID
    bad = rl.FlatPolicy(256, 8, 3, 1)
    assert L.red_max_f32_with(_p(A), 4, _p(B), ctypes.byref(bad), None) == INVALID
    assert L.red_sum_f32_with(_p(A), 4, _p(B), None, None) == INVALID


def test_partials_argument_errors():
    L = rl.lib()
    cnt = ctypes.c_size_t()
    P = 0x40000
    assert L.red_sum_f32_partials(None, 4, _p(P), 8, None, ctypes.byref(cnt), None) == INVALID
    assert L.red_sum_f32_partials(_p(A), 4, None, 8, None, ctypes.byref(cnt), None) == INVALID
    assert L.red_sum_f32_partials(_p(A), 4, _p(P), 8, None, None, None) == INVALID
    assert L.red_sum_f32_partials(_p(A), 4, _p(P + 4), 8, None, ctypes.byref(cnt), None) == INVALID
    bad = rl.FlatPolicy(64, 1, 8, 1, 0, 0, 1)        # grid-stride has no 64-thread blocks
    assert L.red_sum_f32_partials(_p(A), 4, _p(P), 8, ctypes.byref(bad), ctypes.byref(cnt), None) == INVALID
    bad = rl.FlatPolicy(64, 1, 8, 1, 1, 1, 2)        # no combine mode 2
    assert L.red_sum_f32_with(_p(A), 4, _p(B), ctypes.byref(bad), None) == INVALID


def test_default_policies():
    small, mid, big = rl.FlatPolicy(), rl.FlatPolicy(), rl.FlatPolicy()
    rl.lib().red_default_flat_policy(1 << 20, ctypes.byref(small))
    rl.lib().red_default_flat_policy(1 << 24, ctypes.byref(mid))
    rl.lib().red_default_flat_policy(1 << 28, ctypes.byref(big))
    for p in (small, mid, big):
        assert p.layout == 1 and p.combine == 1 and p.nontemporal == 1
    assert big.as_dict() == rl.red_default_flat_policy(1_000_000_007).as_dict()
    r = rl.red_default_rows_policy()
    assert r.block % 64 == 0 and r.max_blocks >= 1


def test_rows_argument_errors():
    L = rl.lib()
    for f in (L.red_rows_sum_f32, L.red_rows_max_f32):
        assert f(_p(A), 1 << 40, 1 << 40, _p(B), None) == INVALID       # rows*cols overflow
        assert f(_p(A), 1 << 21, 1 << 21, _p(B), None) == INVALID       # above RED_MAX_N
        assert f(None, 2, 3, _p(B), None) == INVALID
        assert f(_p(A), 2, 3, None, None) == INVALID
        assert f(_p(A + 2), 2, 3, _p(B), None) == INVALID
        assert f(_p(A), 4, 4, _p(A + 16), None) == INVALID              # out inside x
        assert f(None, 0, 5, None, None) == rl.RED_OK                   # rows == 0: no-op
    bad = rl.RowsPolicy(96, 4, 1, 16, 0)
    assert L.red_rows_sum_f32_with(_p(A), 2, 3, 3, _p(B), ctypes.byref(bad), None) == INVALID
    bad = rl.RowsPolicy(64, 4, 1, 16, 3)
    assert L.red_rows_sum_f32_with(_p(A), 2, 3, 3, _p(B), ctypes.byref(bad), None) == INVALID
    # The fields added for cover reading, the streaming kernel and held results
    # are checked before anything else (rows == 0 then makes a valid call a
    # no-op).
    base = rl.red_default_rows_policy()
    assert base.cover == 0 and base.prefetch == 0 and base.short_rows == 0 and base.defer == 0
    assert base.xcd == 0 and base.max_fold == 0
    for field, value, ok in (("cover", 3, False), ("cover", -1, False), ("cover", 2, True),
                             ("defer", 1, True), ("defer", 2, True), ("defer", 3, False), ("defer", -1, False),
                             ("prefetch", 2, False), ("prefetch", 1, True), ("short_rows", 10, True),
                             ("short_rows", 9, True), ("short_rows", 16, True), ("short_rows", 17, True), ("short_rows", 18, False),
                             ("split", 3, False), ("xcd", -1, False), ("xcd", 1, True), ("xcd", 2, True),
                             ("xcd", 64, True), ("xcd", 4096, True), ("xcd", 4097, False),
                             ("max_fold", 3, False), ("max_fold", -1, False), ("max_fold", 2, True)):
        pol = rl.red_default_rows_policy()
        setattr(pol, field, value)
        want = rl.RED_OK if ok else INVALID
        assert L.red_rows_sum_f32_with(None, 0, 3, 3, None, ctypes.byref(pol), None) == want, (field, value)
    for f in (L.red_rows_sum_f32_ld, L.red_rows_max_f32_ld):
        assert f(_p(A), 2, 5, 4, _p(B), None) == INVALID                   # ld < cols
        assert f(_p(A), 1 << 20, 4, 1 << 21, _p(B), None) == INVALID        # span > RED_MAX_N
        assert f(_p(A), 3, 4, 8, _p(A + 4 * 8), None) == INVALID            # out inside the span
        assert f(None, 0, 4, 8, None, None) == rl.RED_OK


def test_cols_argument_errors():
    L = rl.lib()
    for f in (L.red_cols_sum_f32, L.red_cols_max_f32):
        assert f(_p(A), 2, 5, 4, _p(B), None) == INVALID                 # ld < cols
        assert f(None, 2, 3, 3, _p(B), None) == INVALID
        assert f(_p(A), 2, 3, 3, None, None) == INVALID
        assert f(_p(A + 2), 2, 3, 3, _p(B), None) == INVALID
        assert f(_p(A), 4, 4, 4, _p(A + 16), None) == INVALID           # out inside x
        assert f(_p(A), 1 << 30, 1 << 11, 1 << 11, _p(B), None) == INVALID   # span > RED_MAX_N
        assert f(None, 5, 0, 0, None, None) == rl.RED_OK                 # cols == 0: no-op
    bad = rl.ColsPolicy(3, 1, 1024, 0)
    assert L.red_cols_sum_f32_with(_p(A), 2, 3, 3, _p(B), ctypes.byref(bad), None) == INVALID
    bad = rl.ColsPolicy(8, 1, 1024, 2)
    assert L.red_cols_max_f32_with(_p(A), 2, 3, 3, _p(B), ctypes.byref(bad), None) == INVALID
    base = rl.red_default_cols_policy()
    assert base.fold == 0 and base.vec == 0 and base.order == 0 and base.xcd == 0
    for field, value, ok in (("fold", 65, False), ("fold", -1, False), ("fold", 64, True), ("fold", 17, True), ("fold", 1, True),
                             ("width", 3, False), ("target_waves", 0, False), ("order", 4, False),
                             ("order", -1, False), ("order", 3, True), ("order", 0, True),
                             ("xcd", 3, False), ("xcd", -1, False), ("xcd", 2, True), ("xcd", 1, True)):
        pol = rl.red_default_cols_policy()
        setattr(pol, field, value)
        want = rl.RED_OK if ok else INVALID
        assert L.red_cols_sum_f32_with(None, 5, 0, 0, None, ctypes.byref(pol), None) == want, (field, value)


def test_ablate_argument_errors():
    L = rl.lib()
    assert L.red_ablate_num_partials(1, 1000) == 4
    assert L.red_ablate_num_partials(4, 1000) == 2
    assert L.red_ablate_num_partials(5, 1024) == 2
    assert L.red_ablate_num_partials(9, 1000) == 0
    P = 0x40000
    assert L.red_ablate_sum_f32(0, _p(A), 1000, _p(P), 4, _p(B), None) == INVALID
    assert L.red_ablate_sum_f32(7, _p(A), 1000, _p(P), 4, _p(B), None) == INVALID
    assert L.red_ablate_sum_f32(1, _p(A), 1000, _p(P), 3, _p(B), None) == INVALID   # cap too small
    assert L.red_ablate_sum_f32(1, _p(A), 0, _p(P), 4, _p(B), None) == INVALID
    assert L.red_ablate_sum_f32(2, _p(A), (1 << 31) + 1, _p(P), 1 << 24, _p(B), None) == INVALID
    assert L.red_ablate_sum_f32(3, _p(A), 1000, _p(A + 64), 4, _p(B), None) == INVALID  # overlap
    assert L.red_ablate_sum_f32(6, _p(A), 1000, _p(P), 4, None, None) == INVALID     # rung 6 needs out


def test_probe_argument_errors():
    L = rl.lib()
    assert L.red_probe_copy_f32(_p(A + 4), _p(B), 8, None) == INVALID    # 16-byte alignment
    assert L.red_probe_copy_f32(_p(A), _p(A + 16), 8, None) == INVALID   # overlap
    assert L.red_probe_read_f32(_p(A), 8, None, None) == INVALID
    assert L.red_device_info(None, None, 0) == INVALID
    assert L.red_probe_lds_stride(-2, 1, _p(A), None) == INVALID
    assert L.red_probe_lds_stride(1, -1, _p(A), None) == INVALID
    assert L.red_probe_lds_stride(1, 1, None, None) == INVALID
    assert L.red_probe_wave_reduce(3, _p(A), 1, _p(B), None) == INVALID
    assert L.red_probe_wave_reduce(0, _p(A), 0, _p(B), None) == INVALID
    assert L.red_probe_wave_reduce(0, _p(A + 4), 1, _p(B), None) == INVALID
    assert L.red_probe_wave_reduce(0, _p(A), 2, _p(A + 8), None) == INVALID   # overlap
    assert L.red_probe_shfl_down_f32(_p(A), 65, _p(B), None) == INVALID
    assert L.red_probe_shfl_down_f32(None, 1, _p(B), None) == INVALID
    # The load-only read probe: 16-byte aligned, whole vectors, a shape it compiles.
    sh = rl.red_default_read_shape()
    assert L.red_probe_read_ceiling(_p(A + 4), 64, ctypes.byref(sh), _p(B), None) == INVALID
    assert L.red_probe_read_ceiling(_p(A), 60, ctypes.byref(sh), _p(B), None) == INVALID
    assert L.red_probe_read_ceiling(_p(A), 64, ctypes.byref(sh), None, None) == INVALID
    assert L.red_probe_read_ceiling(_p(A), 64, None, _p(A + 8), None) == INVALID      # sink inside x
    for field, value in (("block", 128), ("unroll", 12), ("layout", 4), ("blocks_per_cu", 0),
                         ("nontemporal", 2)):
        bad = rl.red_default_read_shape()
        setattr(bad, field, value)
        assert L.red_probe_read_ceiling(_p(A), 64, ctypes.byref(bad), _p(B), None) == INVALID, field
    bad = rl.ReadShape(1024, 1, 32, 1, 0)        # would spill: not compiled
    assert L.red_probe_read_ceiling(_p(A), 64, ctypes.byref(bad), _p(B), None) == INVALID
    bad = rl.ReadShape(1024, 1, 16, 1, 2)
    assert L.red_probe_read_ceiling(_p(A), 64, ctypes.byref(bad), _p(B), None) == INVALID
    bad = rl.ReadShape(1024, 1, 16, 1, 3)
    assert L.red_probe_read_ceiling(_p(A), 64, ctypes.byref(bad), _p(B), None) == INVALID


def test_read_shapes_default_is_supported():
    d = rl.red_default_read_shape().as_dict()
    assert d["block"] in (64, 256, 1024) and d["unroll"] in (4, 8, 16, 32) and 0 <= d["layout"] <= 3


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                    reason="only meaningful where no GPU is visible")
def test_no_device():
    L = rl.lib()
    assert L.red_sum_f32(_p(A), 4, _p(B), None) == NO_DEVICE
    assert L.red_last_hip_error() != 0
    assert L.red_rows_max_f32(_p(A), 2, 2, _p(B), None) == NO_DEVICE
    cu = ctypes.c_int()
    assert L.red_device_info(ctypes.byref(cu), None, 0) == NO_DEVICE
    assert L.red_sum_f32_noalloc(_p(A), 4, _p(B), None) == NO_DEVICE
    assert L.red_stream_new_workspace(None) == NO_DEVICE
    assert L.red_probe_fill_workspace(0x7FC00000, None) == NO_DEVICE
    assert L.red_probe_read_ceiling(_p(A), 64, None, _p(B), None) == NO_DEVICE
