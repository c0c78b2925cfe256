#!/usr/bin/env python3
"""Benchmark of libred on one MI355X.

Headline: achieved HBM GB/s of red_sum_f32 over 2^28 float32 elements
(1 GiB, normal(0,1), seed 2), as a fraction of the 8 TB/s HBM3E peak. One
step is one red_sum_f32 call over the resident array: the streaming kernel
(load, peel, wave reduce, LDS combine, block partial) and the one-block
combine launch. The K timed steps are captured in one HIP graph and
replayed once between two events; the same calls launched eagerly are timed
too. The line also carries the roofline of the streaming kernel
(timed alone through red_sum_f32_partials), the CPU oracle timed on the
host, and the other entry points at their own workloads.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
    python bench.py --ablation | --widths | --probe-sweep
                                              (other measurements, one JSON line each)

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0          # MI355X HBM3E peak, 8 TB/s
METRIC = "achieved HBM GB/s (% of MI355X peak) for f32 sum over 2^28 elements"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CPU_THREADS_MAX = 16          # the host CPU share that goes with one GPU
OBJECT_MANIFEST = os.path.join(ROOT, "reduction_libred_amd", "libred_objects.json")
KERNEL_UNIT = "flat_sum_f32.hip"  # the translation unit of the f32 sum kernel


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_identity(policy):
    """Identity of the streaming kernel as launched: the hash of its compiled
    object (from the build's manifest) and the launch shape; None when the
    manifest is missing."""
    try:
        with open(OBJECT_MANIFEST) as fh:
            digest = json.load(fh)[KERNEL_UNIT]
    except (OSError, ValueError, KeyError):
        return None
    h = hashlib.sha256(digest.encode())
    h.update(json.dumps(policy, sort_keys=True).encode())
    return h.hexdigest()


def recorded_traffic(policy):
    """HBM bytes per launch of the sum kernel from the committed counter
    runs, or None if the kernel's code or its launch shape changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ident = kernel_identity(policy)
    if ident is None or rec.get("kernel_identity") != ident:
        return None
    return rec.get("flat_reduce_kernel_sum_f32_2p28_bytes_per_launch")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only: skip the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time budget of the CPU oracle baseline (0 to skip)")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of the headline: time the five-rung ladder and the production "
                         "path on the 2^28 array, and the LDS bank probe; print one JSON line")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="instead of the headline: time the load-only read probe at every launch shape "
                         "on the 2^28-float array and print one JSON line, fastest first")
    ap.add_argument("--combine-sweep", action="store_true",
                    help="instead of the headline: time red_sum_f32 with the second-launch and the "
                         "single-launch (ticket) combine over launch shapes at 2^20, 2^24 and 2^28 elements, "
                         "eager and inside HIP graphs, against the streaming kernel alone; one JSON line")
    ap.add_argument("--widths", action="store_true",
                    help="instead of the headline: time the row and column entry points on 1 GiB "
                         "of f32 viewed as (2^28 // cols) x cols for a range of widths; print one "
                         "JSON line")
    ap.add_argument("--col-orders", action="store_true",
                    help="instead of the headline: time the column entry points on 1 GiB of f32 viewed as "
                         "(2^28 // cols) x cols at widths around the row pitches that alias on the memory "
                         "channels, with each row order and the default; print one JSON line")
    ap.add_argument("--col-strides", action="store_true",
                    help="instead of the headline: time the column entry points on 1 GiB of f32 read as "
                         "rows of ld floats of which the first cols are the matrix, with the default, the "
                         "same launch shape with blocks dealt in launch order instead of grouped per XCD, "
                         "and one column per lane; print one JSON line")
    return ap.parse_args()


# Barriers per 256-thread block, by construction of each rung's kernel: one
# after the LDS store, then one per tree step (8 steps from 256 to 1 for rungs
# 1-4, one step from 256 to 128 for rung 5). The production kernel's default
# 64-thread blocks need none; its combine pass has one.
RUNG_BARRIERS = {1: 9, 2: 9, 3: 9, 4: 9, 5: 2}
RUNG_NAMES = {1: "interleaved, divergent", 2: "interleaved, strided (bank conflicts)",
              3: "sequential addressing", 4: "first add during load", 5: "wave64 shuffle finish",
              6: "production (wave tiles + DPP)"}
LDS_STRIDES = [1, 2, 4, 8, 16, 32, 64, 128, 3, 33, 65, 0, -1]


def run_ablation(args, torch, rl, W, timer, dev):
    name = "sum_max_f32_2p28"
    log(f"generate {name}")
    x = torch.from_numpy(W.workload(name)).to(dev)
    n = x.numel()
    rungs = []
    out = torch.empty((), dtype=torch.float32, device=dev)
    for rung in range(1, 6):
        np_ = rl.red_ablate_num_partials(rung, n)
        partials = torch.empty(np_, dtype=torch.float32, device=dev)

        def kern():
            rl.red_ablate_sum_f32(rung, x, partials=partials, partials_only=True)

        for _ in range(args.warmup):
            kern()
        ms = timer.region_ms(kern, args.steps)
        rl.red_ablate_sum_f32(rung, x, partials=partials, out=out)
        torch.cuda.synchronize()
        rungs.append({"rung": rung, "what": RUNG_NAMES[rung], "blocks": np_, "block_threads": 256,
                      "barriers_per_block": RUNG_BARRIERS[rung], "kernel_us": round(ms * 1e3, 2),
                      "GB/s": round(gbps(4 * n, ms), 1), "pct_of_peak": round(100 * gbps(4 * n, ms) / PEAK_GBPS, 2),
                      "sum": out.item()})
        log(f"rung {rung}: {rungs[-1]}")
        del partials
    pol = rl.red_default_flat_policy(n).as_dict()
    grid = rl.red_flat_grid(n)
    parts = torch.empty(grid, dtype=torch.float64, device=dev)
    kern6 = lambda: rl.red_sum_f32_partials(x, partials=parts)
    for _ in range(args.warmup):
        kern6()
    ms = timer.region_ms(kern6, args.steps)
    rl.red_sum_f32(x, out=out)
    torch.cuda.synchronize()
    rungs.append({"rung": 6, "what": RUNG_NAMES[6], "blocks": grid, "block_threads": pol["block"],
                  "barriers_per_block": 0 if pol["block"] == 64 else 1, "kernel_us": round(ms * 1e3, 2),
                  "GB/s": round(gbps(4 * n, ms), 1), "pct_of_peak": round(100 * gbps(4 * n, ms) / PEAK_GBPS, 2),
                  "sum": out.item(), "policy": pol})
    log(f"rung 6: {rungs[-1]}")
    del x
    probe = []
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    iters = 4096
    rl.red_probe_lds_stride(1, iters, sink)          # load the kernel before timing
    for stride in LDS_STRIDES:
        ms = timer.region_ms(lambda: rl.red_probe_lds_stride(stride, iters, sink), 5)
        probe.append({"stride": stride, "us_per_launch": round(ms * 1e3, 2),
                      "ns_per_read": round(ms * 1e6 / iters, 3)})
        log(f"lds stride {stride}: {probe[-1]}")
    print(json.dumps({"mode": "ablation", "workload": name, "n": n, "steps": args.steps,
                      "rungs": rungs, "lds_probe": {"iters": iters, "words": 64 * 65, "strides": probe}}),
          flush=True)


# Row lengths covering each row and column path: one float, odd widths (the
# LDS-staged rows, folded column views), multiples of 4 (packed and staged
# rows, four columns per lane), and long rows (one wave per row; odd lengths
# read through their aligned covers).
WIDTHS = [1, 3, 4, 7, 12, 16, 17, 24, 32, 33, 64, 65, 100, 256, 260, 512, 1000, 1020, 1023, 1025, 2049, 4096,
          4097, 6000, 16385, 50257]


def run_widths(args, torch, rl, W, timer, dev):
    name = "rows_f32_65536x4096"
    log(f"generate {name}")
    flat = torch.from_numpy(W.workload(name)).to(dev).view(-1)
    total = flat.numel()
    shapes = []
    for cols in WIDTHS:
        rows = total // cols
        m = flat[: rows * cols].view(rows, cols)
        ro = torch.empty(rows, device=dev)
        co = torch.empty(cols, device=dev)
        entry = {"rows": rows, "cols": cols}
        calls = (("rows_sum", lambda: rl.red_rows_sum_f32(m, out=ro), rows),
                 ("rows_max", lambda: rl.red_rows_max_f32(m, out=ro), rows),
                 ("cols_sum", lambda: rl.red_cols_sum_f32(m, out=co), cols),
                 ("cols_max", lambda: rl.red_cols_max_f32(m, out=co), cols))
        for label, fn, nout in calls:
            for _ in range(args.warmup):
                fn()
            ms = timer.region_ms(fn, args.steps)
            nin = 4 * rows * cols
            entry[label] = {"us": round(ms * 1e3, 2), "GB/s": round(gbps(nin, ms), 1),
                            "GB/s_with_output": round(gbps(nin + 4 * nout, ms), 1),
                            "pct_of_peak": round(100 * gbps(nin, ms) / PEAK_GBPS, 2)}
        log(f"{rows}x{cols}: " + ", ".join(f"{k} {entry[k]['GB/s']}" for k in ("rows_sum", "rows_max",
                                                                                 "cols_sum", "cols_max")))
        shapes.append(entry)
    print(json.dumps({"mode": "widths", "workload": f"{name} viewed as (2^28 // cols) x cols, contiguous",
                      "steps": args.steps, "warmup": args.warmup, "unit": "GB/s of input",
                      "shapes": shapes}), flush=True)


# Widths whose rows (or 32-row views) have a pitch that is a multiple of 255
# or 257 floats, and neighbours that are not; then narrow matrices whose wave
# loads cover several rows, with and without whole 128-byte lines per load.
ORDER_WIDTHS = [1016, 1020, 1024, 1028, 2040, 2044, 3060, 4080, 5100, 8160, 765, 4096, 3, 4, 12, 16, 17, 24]
COL_ORDERS = (("band", dict(order=1)), ("rotated", dict(order=2)), ("chunks", dict(order=3)), ("default", None))


def run_col_orders(args, torch, rl, W, timer, dev):
    name = "rows_f32_65536x4096"
    log(f"generate {name}")
    flat = torch.from_numpy(W.workload(name)).to(dev).view(-1)
    total = flat.numel()
    shapes = []
    for cols in ORDER_WIDTHS:
        rows = total // cols
        m = flat[: rows * cols].view(rows, cols)
        co = torch.empty(cols, device=dev)
        entry = {"rows": rows, "cols": cols}
        for op_name, op in (("sum", rl.red_cols_sum_f32), ("max", rl.red_cols_max_f32)):
            for label, pol in COL_ORDERS:
                def fn():
                    op(m, out=co, policy=pol)
                for _ in range(args.warmup):
                    fn()
                ms = timer.region_ms(fn, args.steps)
                entry[f"{op_name}_{label}"] = round(gbps(4 * rows * cols, ms), 1)
        log(f"{rows}x{cols}: " + ", ".join(f"{k} {v}" for k, v in entry.items() if k not in ("rows", "cols")))
        shapes.append(entry)
    print(json.dumps({"mode": "col_orders", "workload": f"{name} viewed as (2^28 // cols) x cols, contiguous",
                      "steps": args.steps, "warmup": args.warmup, "unit": "GB/s of input",
                      "orders": [k for k, _ in COL_ORDERS], "shapes": shapes}), flush=True)


# Strided matrices: rows that start 4-byte but not 16-byte aligned (odd ld),
# and two 16-byte aligned pitches that are not whole lines (4100, 1028).
STRIDE_SHAPES = [(4096, 4097), (4096, 4100), (8192, 8193), (3000, 3001), (2000, 2001), (1020, 1021), (1024, 1028),
                 (500, 503), (300, 301), (256, 257), (200, 201), (128, 129), (100, 101), (64, 65), (33, 35),
                 (17, 19), (12, 13), (5, 7)]


def stride_variants(cols, ld):
    """The library's default for a (cols, ld) matrix at an aligned x, the
    same launch shape with blocks dealt in launch order (xcd 1), and the
    one-column-per-lane shape that was the default for such rows before the
    shifted-vector form."""
    if ld % 4 == 0 and cols % 4 == 0:
        same = dict(xcd=1)
    elif (cols + 3) // 4 + (cols % 4 != 1) >= 64:  # a spare group makes 64 lanes a row
        same = dict(unroll=4, width=2, target_waves=1024, prefetch=1, xcd=1)
    else:
        same = dict(unroll=8, width=1, target_waves=2048, prefetch=1, xcd=1)
    return (("default", None), ("launch_order", same),
            ("one_per_lane", dict(vec=1, unroll=8, width=2, target_waves=2048, prefetch=0, xcd=1)))


def run_col_strides(args, torch, rl, W, timer, dev):
    name = "rows_f32_65536x4096"
    log(f"generate {name}")
    flat = torch.from_numpy(W.workload(name)).to(dev).view(-1)
    total = flat.numel()
    shapes = []
    for cols, ld in STRIDE_SHAPES:
        rows = total // ld
        m = flat[: rows * ld].view(rows, ld)[:, :cols]
        co = torch.empty(cols, device=dev)
        entry = {"rows": rows, "cols": cols, "ld": ld}
        for op_name, op in (("sum", rl.red_cols_sum_f32), ("max", rl.red_cols_max_f32)):
            for label, pol in stride_variants(cols, ld):
                def fn():
                    op(m, out=co, policy=pol)
                for _ in range(args.warmup):
                    fn()
                ms = timer.region_ms(fn, args.steps)
                entry[f"{op_name}_{label}"] = round(gbps(4 * rows * cols, ms), 1)
        log(f"{rows}x{cols} ld {ld}: " + ", ".join(f"{k} {v}" for k, v in entry.items()
                                                  if k not in ("rows", "cols", "ld")))
        shapes.append(entry)
    print(json.dumps({"mode": "col_strides", "workload": f"{name} read as (2^28 // ld) rows of ld floats, "
                      "the first cols of each the matrix", "steps": args.steps, "warmup": args.warmup,
                      "unit": "GB/s of matrix bytes (4 * rows * cols)",
                      "variants": [k for k, _ in stride_variants(1, 1)], "shapes": shapes}), flush=True)


def read_shapes():
    """Every launch shape of the read probe: block 64 / 256 / 1024, 1-16 waves
    per CU, 4-32 loads in flight per lane, non-temporal or not, four layouts
    (the shapes that fit in registers without spilling)."""
    for block in (64, 256, 1024):
        per_block = block // 64
        for waves in (1, 2, 4, 8, 16):
            if waves < per_block or waves % per_block:
                continue
            for unroll in (4, 8, 16, 32):
                for layout in (0, 1, 2, 3):
                    if block == 1024 and (unroll > 16 or (layout >= 2 and unroll > 8)):
                        continue
                    for nt in (0, 1):
                        yield dict(block=block, blocks_per_cu=waves // per_block, unroll=unroll, nontemporal=nt,
                                   layout=layout)


def run_probe_sweep(args, torch, rl, W, timer, dev):
    name = "sum_max_f32_2p28"
    log(f"generate {name}")
    x = torch.from_numpy(W.workload(name)).to(dev)
    nbytes = 4 * x.numel()
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    results = []
    reps = max(5, min(args.steps, 30))
    for shape in read_shapes():
        fn = lambda: rl.red_probe_read_ceiling(x, sink=sink, shape=shape)
        for _ in range(3):
            fn()
        ms = timer.region_ms(fn, reps)
        results.append(dict(shape, **{"us": round(ms * 1e3, 2), "GB/s": round(gbps(nbytes, ms), 1)}))
        log(f"{shape}: {results[-1]['GB/s']} GB/s")
    results.sort(key=lambda r: -r["GB/s"])
    # The five fastest again, alternating, to separate them from noise.
    top = results[:5]
    again = {i: [] for i in range(len(top))}
    for _ in range(3):
        for i, r in enumerate(top):
            shape = {k: r[k] for k in ("block", "blocks_per_cu", "unroll", "nontemporal", "layout")}
            ms = timer.region_ms(lambda: rl.red_probe_read_ceiling(x, sink=sink, shape=shape), reps)
            again[i].append(gbps(nbytes, ms))
    for i, r in enumerate(top):
        r["GB/s_rerun_median"] = round(sorted(again[i])[1], 1)
    # The copy probe (reads and writes) at its shapes: the ceiling for a
    # reduction whose output is as large as its input.
    y = torch.empty_like(x)
    copies = []
    for bpc in (1, 2, 4, 8):
        for unroll in (4, 8, 16):
            for nt in (0, 1):
                shape = dict(block=64, blocks_per_cu=bpc, unroll=unroll, nontemporal=nt, layout=2)
                fn = lambda: rl.red_probe_copy_ceiling(x, y, shape=shape)
                for _ in range(3):
                    fn()
                ms = timer.region_ms(fn, reps)
                copies.append(dict(shape, **{"us": round(ms * 1e3, 2), "GB/s_read_plus_write": round(gbps(2 * nbytes, ms), 1)}))
                log(f"copy {shape}: {copies[-1]['GB/s_read_plus_write']} GB/s")
    copies.sort(key=lambda r: -r["GB/s_read_plus_write"])
    del y
    # The reduction kernel in the same process, for comparison.
    parts = torch.empty(rl.red_flat_grid(x.numel()), dtype=torch.float64, device=dev)
    for _ in range(3):
        rl.red_sum_f32_partials(x, partials=parts)
    ms = timer.region_ms(lambda: rl.red_sum_f32_partials(x, partials=parts), reps)
    print(json.dumps({"mode": "probe_sweep", "workload": name, "bytes": nbytes, "reps": reps,
                      "default_shape": rl.red_default_read_shape().as_dict(),
                      "sum_kernel_GB/s": round(gbps(nbytes + 4, ms), 1), "shapes": results,
                      "copy_default_shape": rl.red_default_copy_shape().as_dict(), "copy_shapes": copies}), flush=True)


COMBINE_SHAPES = [(64, 2, 8), (64, 1, 8), (256, 1, 8), (256, 1, 4), (1024, 1, 4), (1024, 1, 8)]


def run_combine_sweep(args, torch, rl, W, timer, dev):
    """Both forms of the final combine: a one-wave second launch (combine 1)
    and the ticket, where the last block to finish combines (combine 0),
    which needs an agent-scope release by every block before its counter
    update."""
    stream = torch.cuda.current_stream(dev)
    rows = []
    for n in (1 << 20, 1 << 24, 1 << 28):
        log(f"generate normal n={n}")
        x = torch.from_numpy(W.make("normal", n, 2)).to(dev)
        out = torch.empty((), device=dev)
        reps = 50 if n >= 1 << 28 else 200
        for (b, bpc, u) in COMBINE_SHAPES:
            for comb in (1, 0):
                pol = dict(block=b, blocks_per_cu=bpc, unroll=u, layout=1, prefetch=1, nontemporal=1, combine=comb)
                fn = lambda: rl.red_sum_f32(x, out=out, policy=pol)
                for _ in range(5):
                    fn()
                eager = timer.region_ms(fn, reps)
                cap = torch.cuda.Stream()
                cap.wait_stream(stream)
                with torch.cuda.stream(cap):
                    fn()
                    torch.cuda.synchronize()
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=cap):
                        for _ in range(50):
                            rl.red_sum_f32(x, out=out, policy=pol)
                torch.cuda.synchronize()
                g.replay()
                graph = timer.region_ms(g.replay, 10) / 50
                parts = rl.red_sum_f32_partials(x, policy=pol)
                kfn = lambda: rl.red_sum_f32_partials(x, partials=parts, policy=pol)
                for _ in range(5):
                    kfn()
                kern = timer.region_ms(kfn, reps)
                rows.append(dict(n=n, block=b, blocks_per_cu=bpc, unroll=u, combine=comb,
                                 grid=rl.red_flat_grid(n, pol), eager_us=round(eager * 1e3, 3),
                                 graph_us=round(graph * 1e3, 3), kernel_alone_us=round(kern * 1e3, 3)))
                log(json.dumps(rows[-1]))
                del g
        del x
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "combine_sweep", "workload": "normal(0,1) float32, seed 2", "rows": rows}),
          flush=True)


class Timer:
    """HIP events on one stream around a region of `reps` enqueued calls."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def region_ms(self, fn, reps):
        t = self.torch
        e0 = t.cuda.Event(enable_timing=True)
        e1 = t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(reps):
            fn()
        e1.record(self.stream)
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def per_launch_ms(self, fn, reps):
        t = self.torch
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(reps)]
        t.cuda.synchronize()
        for a, b in ev:
            a.record(self.stream)
            fn()
            b.record(self.stream)
        t.cuda.synchronize()
        d = sorted(a.elapsed_time(b) for a, b in ev)
        return d[len(d) // 2], d[0]


def gbps(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the library "
              "reduces on one GPU, and sharding across GPUs is not implemented.", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    import reduction_libred_amd as rl

    if not os.path.exists(rl.LIB_PATH):
        from reduction_libred_amd import build as lib_build
        lib_build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    timer = Timer(torch, stream)
    cu, arch = rl.red_device_info()
    log(f"device: {torch.cuda.get_device_name(dev)} {arch}, {cu} CUs; {rl.red_version()}")
    if args.ablation:
        run_ablation(args, torch, rl, W, timer, dev)
        return
    if args.widths:
        run_widths(args, torch, rl, W, timer, dev)
        return
    if args.probe_sweep:
        run_probe_sweep(args, torch, rl, W, timer, dev)
        return
    if args.col_orders:
        run_col_orders(args, torch, rl, W, timer, dev)
        return
    if args.col_strides:
        run_col_strides(args, torch, rl, W, timer, dev)
        return
    if args.combine_sweep:
        run_combine_sweep(args, torch, rl, W, timer, dev)
        return

    # ---------------------------------------------------------- headline
    name = "sum_max_f32_2p28"
    log(f"generate {name}")
    a = W.workload(name)
    n = a.size
    x = torch.from_numpy(a).to(dev)
    out = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    policy = rl.red_default_flat_policy(n).as_dict()
    grid = rl.red_flat_grid(n)
    nbytes = 4 * n + 4

    def step():
        rl.red_sum_f32(x, out=out)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager = out.item()
    log(f"timed {args.steps} eager steps")
    ms_eager = timer.region_ms(step, args.steps)
    if out.item() != eager:
        raise RuntimeError("red_sum_f32 is not reproducible run to run")
    log(f"red_sum_f32 eager: {ms_eager * 1e3:.1f} us/step, {gbps(nbytes, ms_eager):.1f} GB/s")
    # Each eager step bracketed by its own events: median and min.
    step_med, step_min = timer.per_launch_ms(step, max(20, min(args.steps, 200)))

    # The timed steps: the same K calls captured in one HIP graph (launch
    # overhead out of the way, as a serving loop would run them), replayed
    # once between two events. The capture stream gets its workspace from an
    # eager call first; the replay must give the eager bits.
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(args.steps):
                step()
    torch.cuda.synchronize()
    out.zero_()
    graph.replay()                              # warm
    torch.cuda.synchronize()
    if out.item() != eager:
        raise RuntimeError("graph replay of red_sum_f32 differs from the eager result")
    log(f"timed {args.steps} steps in one graph replay")
    ms = timer.region_ms(graph.replay, 1) / args.steps
    if out.item() != eager:
        raise RuntimeError("graph replay of red_sum_f32 differs from the eager result")
    value = gbps(nbytes, ms)
    log(f"red_sum_f32: {ms * 1e3:.1f} us/step, {value:.1f} GB/s ({100 * value / PEAK_GBPS:.1f}% of peak)")
    replays = sorted(timer.region_ms(graph.replay, 1) / args.steps for _ in range(5))
    del graph

    # The dominant kernel alone: steps 1-5 (the streaming pass) without the
    # one-block combine launch, via red_sum_f32_partials, same launch shape.
    partials = torch.empty(grid, dtype=torch.float64, device=dev)

    def pass1():
        rl.red_sum_f32_partials(x, partials=partials)

    for _ in range(args.warmup):
        pass1()
    k_ms = timer.region_ms(pass1, args.steps)
    med_ms, min_ms = timer.per_launch_ms(pass1, max(20, min(args.steps, 200)))
    achieved = gbps(nbytes, k_ms)
    log(f"flat_reduce_kernel alone: {k_ms * 1e3:.1f} us/launch, {achieved:.1f} GB/s; "
        f"per-launch median {med_ms * 1e3:.1f} us")
    # The achievable read ceiling: the load-only probe at its default (the
    # fastest swept) shape over the same resident array.
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    probe = lambda: rl.red_probe_read_ceiling(x, sink=sink)
    for _ in range(args.warmup):
        probe()
    p_ms = timer.region_ms(probe, args.steps)
    p_med, p_min = timer.per_launch_ms(probe, max(20, min(args.steps, 200)))
    probe_gbps = gbps(4 * n, p_ms)
    log(f"read probe: {p_ms * 1e3:.1f} us/launch, {probe_gbps:.1f} GB/s")
    kname = (f"flat_reduce_kernel<SumF32, {policy['block']}, {policy['unroll']}, "
             f"{'true' if policy['nontemporal'] else 'false'}, {policy['layout']}, "
             f"{'true' if policy['prefetch'] else 'false'}>")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": "sum_max_f32_2p28: float32 sum of 2^28 elements (1 GiB), normal(0,1), seed 2",
            "n": n,
            "entry_point": "red_sum_f32",
            "input_dtype": "f32",
            "accumulate_dtype": "f64",
            "policy": policy,
            "grid": grid,
            "device": arch,
            "cus": cu,
        },
        "pct_of_peak": round(100 * value / PEAK_GBPS, 2),
        "pct_of_probe": round(100 * value / probe_gbps, 2),
        "elements_per_s": round(n / (ms * 1e-3), 1),
        "timing": f"{args.steps} red_sum_f32 calls captured in one HIP graph, one replay between two HIP "
                  "events on the stream; eager = the same calls launched one by one",
        "step_us": {"graph_mean": round(ms * 1e3, 3),
                    "graph_median_of_5_replays": round(replays[2] * 1e3, 3),
                    "graph_min_of_5_replays": round(replays[0] * 1e3, 3),
                    "eager_mean": round(ms_eager * 1e3, 3), "eager_median": round(step_med * 1e3, 3),
                    "eager_min": round(step_min * 1e3, 3), "eager_GB/s": round(gbps(nbytes, ms_eager), 2),
                    "eager_median_GB/s": round(gbps(nbytes, step_med), 2)},
        "read_ceiling": {"kernel": "read_probe_kernel (load-only, xor of every word)",
                         "shape": rl.red_default_read_shape().as_dict(), "us": round(p_ms * 1e3, 3),
                         "median_us": round(p_med * 1e3, 3), "min_us": round(p_min * 1e3, 3),
                         "GB/s": round(probe_gbps, 2), "pct_of_peak": round(100 * probe_gbps / PEAK_GBPS, 2),
                         "kernel_pct_of_probe": None},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": recorded_traffic(policy),
            "kernel": kname,
            "algorithmic_bytes_per_launch": nbytes,
            "avg_launch_us": round(k_ms * 1e3, 3),
            "median_launch_us_events": round(med_ms * 1e3, 3),
            "min_launch_us_events": round(min_ms * 1e3, 3),
            "step_us_with_combine_launch": round(ms * 1e3, 3),
            "step_over_kernel": round(ms / k_ms, 4),
        },
    }

    result["read_ceiling"]["kernel_pct_of_probe"] = round(100 * achieved / probe_gbps, 2)

    # ---------------------------------------------------------- other entry points
    others = {}
    reps = 50  # calls per timed region; each line is the median of three regions

    def measure(label, fn, nbytes_call, extra=None):
        for _ in range(10):
            fn()
        t_ms = sorted(timer.region_ms(fn, reps) for _ in range(3))[1]
        rec = {"us": round(t_ms * 1e3, 3), "GB/s": round(gbps(nbytes_call, t_ms), 2),
               "pct_of_peak": round(100 * gbps(nbytes_call, t_ms) / PEAK_GBPS, 2)}
        if extra:
            rec.update(extra)
        others[label] = rec
        log(f"{label}: {rec}")

    mout = torch.empty((), dtype=torch.float32, device=dev)
    measure("red_max_f32 sum_max_f32_2p28", lambda: rl.red_max_f32(x, out=mout), nbytes)
    fout = torch.empty(3, dtype=torch.float32, device=dev)
    measure("red_sum_max_f32 (fused sum, max, sum|x|) sum_max_f32_2p28",
            lambda: rl.red_sum_max_f32(x, out=fout), 4 * n + 12)
    measure("red_min_f32 sum_max_f32_2p28", lambda: rl.red_min_f32(x, out=mout), nbytes)
    iout = torch.empty((), dtype=torch.int64, device=dev)
    measure("red_argmax_f32 sum_max_f32_2p28", lambda: rl.red_argmax_f32(x, out=iout), 4 * n + 8)
    # The int32 sum over 1 GiB: the same 2^28 words read as int32 (their bit
    # patterns; every value is exact in the int64 accumulator).
    measure("red_sum_i32_i64 2^28 int32 (1 GiB, the bits of the normal array)",
            lambda: rl.red_sum_i32_i64(x.view(torch.int32), out=iout), 4 * n + 8)
    if not args.quick:
        # The same 2^28 values rounded to 16-bit formats (2^29 elements = 1 GiB
        # after doubling the count) and a 1 GiB float64 array.
        for tdt, fn, label in ((torch.bfloat16, rl.red_sum_bf16_f32, "red_sum_bf16_f32"),
                               (torch.float16, rl.red_sum_f16_f32, "red_sum_f16_f32")):
            xh = torch.cat([x, x]).to(tdt)
            measure(f"{label} 2^29 elements (1 GiB, the 2^28 normal array twice)",
                    lambda: fn(xh, out=mout), 2 * xh.numel() + 4)
            del xh
        xd = x[: n // 2].to(torch.float64)
        dout = torch.empty((), dtype=torch.float64, device=dev)
        measure("red_sum_f64 2^27 elements (1 GiB)", lambda: rl.red_sum_f64(xd, out=dout), 8 * xd.numel() + 8)
        del xd
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    measure("probe read sum_max_f32_2p28", lambda: rl.red_probe_read_f32(x, sink=sink), 4 * n)
    y = torch.empty_like(x)
    measure("probe copy sum_max_f32_2p28", lambda: rl.red_probe_copy_f32(x, y), 8 * n)
    measure("probe copy ceiling (default shape) sum_max_f32_2p28, read plus write bytes",
            lambda: rl.red_probe_copy_ceiling(x, y), 8 * n)
    del y

    if not args.quick:
        # Rows: 65536 x 4096.
        name4 = "rows_f32_65536x4096"
        log(f"generate {name4}")
        x4 = torch.from_numpy(W.workload(name4)).to(dev)
        r4 = torch.empty(x4.shape[0], dtype=torch.float32, device=dev)
        b4 = 4 * x4.numel() + 4 * x4.shape[0]
        measure(f"red_rows_sum_f32 {name4}", lambda: rl.red_rows_sum_f32(x4, out=r4), b4)
        measure(f"red_rows_max_f32 {name4}", lambda: rl.red_rows_max_f32(x4, out=r4), b4)
        c4 = torch.empty(x4.shape[1], dtype=torch.float32, device=dev)
        bc = 4 * x4.numel() + 4 * x4.shape[1]
        measure(f"red_cols_sum_f32 {name4}", lambda: rl.red_cols_sum_f32(x4, out=c4), bc)
        measure(f"red_cols_max_f32 {name4}", lambda: rl.red_cols_max_f32(x4, out=c4), bc)
        del x4

        # Small, cache-resident sizes, through HIP graphs so that host call
        # overhead is out of the measurement: "batched" replays 100 calls on
        # one array (it stays in the 256 MB Infinity Cache); "cold" replays
        # calls that rotate over copies totalling 1 GiB, so each call's input
        # was evicted by the others. Replays are checked against the eager
        # result.
        for name_s, fn_s, odt in (("sum_f32_2p20", rl.red_sum_f32, torch.float32),
                                  ("sum_i32_2p24", rl.red_sum_i32_i64, torch.int64)):
            log(f"generate {name_s}")
            xs = torch.from_numpy(W.workload(name_s)).to(dev)
            os_ = torch.empty((), dtype=odt, device=dev)
            bs = xs.element_size() * xs.numel() + os_.element_size()
            fn_s(xs, out=os_)
            torch.cuda.synchronize()
            eager_s = os_.item()
            copies = max(2, -(-(1 << 30) // (bs - os_.element_size())))
            xc = [xs.clone() for _ in range(copies)]
            rec = {}
            for label, inputs in (("batched", [xs] * 100), ("cold", xc)):
                g = torch.cuda.CUDAGraph()
                cap = torch.cuda.Stream()
                cap.wait_stream(stream)
                with torch.cuda.stream(cap):
                    fn_s(xs, out=os_)      # the capture stream's workspace exists before capture
                    torch.cuda.synchronize()
                    with torch.cuda.graph(g, stream=cap):
                        for xi in inputs:
                            fn_s(xi, out=os_)
                torch.cuda.synchronize()
                for _ in range(3):
                    os_.zero_()
                    g.replay()
                    torch.cuda.synchronize()
                    if os_.item() != eager_s:
                        raise RuntimeError(f"graph replay of {name_s} differs from the eager result")
                t_ms = timer.region_ms(g.replay, 10) / len(inputs)
                rec[f"{label}_us"] = round(t_ms * 1e3, 3)
                rec[f"{label}_GB/s"] = round(gbps(bs, t_ms), 2)
                del g
            rec["note"] = ("fits in the 256 MB Infinity Cache; batched = 100 calls on one array in a HIP graph, "
                           f"cold = {copies} calls on distinct copies (1 GiB in all) in a HIP graph")
            others[f"{fn_s.__name__} {name_s}"] = rec
            log(f"{fn_s.__name__} {name_s}: {rec}")
            del xc, xs
            torch.cuda.empty_cache()

        name5 = "sum_f32_1e9p7"
        log(f"generate {name5}")
        a5 = W.workload(name5)
        x5 = torch.from_numpy(a5).to(dev)
        del a5
        o5 = torch.empty((), dtype=torch.float32, device=dev)
        measure(f"red_sum_f32 {name5}", lambda: rl.red_sum_f32(x5, out=o5), 4 * x5.numel() + 4)
        del x5
        torch.cuda.empty_cache()
    result["other_entry_points"] = others

    # ---------------------------------------------------------- CPU oracle
    if args.cpu_seconds > 0:
        import oracle

        def time_oracle(fn, budget):
            passes, t0 = 0, time.perf_counter()
            while True:
                fn(a)
                passes += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    return passes, el

        threads = max(1, min(len(os.sched_getaffinity(0)), CPU_THREADS_MAX))
        log(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s: {threads} threads, then 1)")
        p_mt, el_mt = time_oracle(lambda v: oracle.sum_f32_mt(v, threads), args.cpu_seconds / 2)
        p_st, el_st = time_oracle(oracle.sum_f32, args.cpu_seconds / 2)
        result["cpu_baseline"] = {
            "value": round(gbps(nbytes * p_mt, el_mt * 1e3), 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{p_mt} full pass(es) of the oracle's chunked float64 Neumaier sum on {threads} host "
                      f"threads over the same 2^28-element host array, {el_mt:.1f} s",
            "elements_per_s": round(n * p_mt / el_mt, 1),
            "single_thread": {
                "value": round(gbps(nbytes * p_st, el_st * 1e3), 3),
                "unit": "GB/s",
                "cores": 1,
                "sample": f"{p_st} full pass(es) of the single-threaded oracle, {el_st:.1f} s",
                "elements_per_s": round(n * p_st / el_st, 1),
            },
            "host_cpu": _cpu_model(),
            "host_threads": os.cpu_count(),
        }
    print(json.dumps(result), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
