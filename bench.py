#!/usr/bin/env python3
"""Throughput of the device-wide chained scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the library entry point over the whole input resident
in HBM (one kernel launch on a prepared workspace).  W untimed steps, then K
steps timed with the wall clock between two device synchronisations; HIP
events that the library records around its main kernel on the same stream,
on every 5th of those steps, give that kernel's average duration for the
roofline figure.  Then, outside those K steps: R more calls, each after a
flush of the caches (1 GiB read and written through a scratch tensor, four
times the 256 MB MALL), timed one by one with HIP events (median, min,
max); and, in the same process and under both protocols, the plain copy,
read and write streams of 1 GiB, and a plain stream with the workload's
own mix of read and written bytes, that set the practical ceiling
(`stream_ceiling`).  Prints one JSON line.

Workloads (default: u32x): the headline is the uint32 exclusive sum scan of
2^28 elements, values uniform in [0, 255] (seed 2).  The others time the
remaining kernels on their configurations:
  u32x-ragged  same, n = 2^28 - 12345            u32i  inclusive, n = 2^28
  f32          fp32 inclusive sum, n = 2^27, N(0,1)  f32max  fp32 inclusive max
  segmented    segmented u32 exclusive, 2^26 values, 2^16 Zipf(1.2) segments
  compact      2^26 16-byte records, Bernoulli(0.3) keep flags
  compact-staged  the same as two passes (flag scan, then scatter): the
               ablation of the fused kernel
  u64x         widening u32 -> u64 exclusive sum scan, n = 2^28 (12 B/element)
  u32s         the small configuration, n = 2^20 values in [0, 15] (seed 1),
               through the default entry point (its two-level form)
  u32s-single-pass   the same with the single-pass form forced
  linrec       linear recurrence h = a h + b as an inclusive fp32 pair scan,
               n = 2^27 pairs in two planes, both outputs (16 B/pair)
  linrec-h     the same, only B = h written (12 B/pair)
  copy         plain 1 GiB copy (the practical bandwidth ceiling)
  read, write  its halves: 1 GiB only read, 1 GiB only written

Only the cpu_baseline leg runs the oracle: the sequential C scan, one host
thread, timed on the same input, and its output is compared with the GPU's.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
METRIC = "Gelem/s and % of HBM peak GB/s, 2^28 uint32 exclusive scan on 1 MI355X"
PROFILES = os.path.join(ROOT, "profiles")
# The kernel time comes from HIP event pairs on a sample of the timed steps:
# every 5th main-kernel launch (odd, so the two kernels of a two-kernel step
# are sampled alike).  Each timed launch carries two event packets (a few µs),
# which a sample spreads over the wall-clock steps.
TIMING_EVERY = 5


# The source file that holds each workload's main kernel (scan.hip for the
# rest); its hash, with every shared header, marks the counter summaries under
# profiles/ taken on it, so that a change to one kernel leaves the others'
# summaries valid.
KERNEL_FILE = {"segmented": "segscan.hip", "compact": "compact.hip",
               "copy": "common.hip", "read": "common.hip", "write": "common.hip"}


def kernel_sources(workload: str):
    csrc = os.path.join(ROOT, "device_wide_prefix_chained_amd", "csrc")
    files = [os.path.join(csrc, KERNEL_FILE.get(workload, "scan.hip"))]
    files += sorted(glob.glob(os.path.join(csrc, "*.hpp")))
    files.append(os.path.join(ROOT, "include", "dwps.h"))
    return files


def _code_text(text: str) -> str:
    """The source with its comments removed and its whitespace collapsed,
    so that a change to comments alone keeps the hash.  A string literal is
    kept whole, so that a comment marker inside one is not taken for a
    comment."""
    token = re.compile(r'"(?:\\.|[^"\\])*"|//[^\n]*|/\*.*?\*/', re.S)
    text = token.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return " ".join(text.split())


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for p in kernel_sources(workload):
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(_code_text(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, launch_bytes_alg: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, or None when absent or taken on different kernel sources."""
    path = os.path.join(PROFILES, "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash(workload):
        return None
    return float(t["hbm_bytes_per_launch"])


def build_workload(name: str):
    """Return (description, dtype, n, algorithmic bytes per call, host inputs, runner factory)."""
    import torch

    import device_wide_prefix_chained_amd as dw
    import workloads as wl

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint32:
            a = a.view(np.int32)
        return torch.from_numpy(a).to("cuda")

    if name in ("u32s", "u32s-single-pass"):
        # the small configuration: the flat entry point runs its two-level
        # form here; the second name forces the single-pass form for contrast
        n = wl.N_SMALL_U32
        x = wl.small_u32()
        d_in, d_out = dev(x), torch.empty(n, dtype=torch.int32, device="cuda")
        if name == "u32s":
            ws = dw.new_workspace(dw.workspace_bytes("ps_scan_exclusive_u32", None, None, n, None, None))
            run = lambda: dw.ps_scan_exclusive_u32(d_in, d_out, workspace=ws)  # noqa: E731
            form = "default entry point (two-level form at this size)"
        else:
            ws = dw.new_workspace(dw.workspace_bytes("ps_scan_single_pass", 0, 0, 0, None, None, n, None, None))
            run = lambda: dw.ps_scan_single_pass("sum", False, d_in, d_out, workspace=ws)  # noqa: E731
            form = "single-pass form forced"
        tile = dw.ps_two_level_tile_elements() if name == "u32s" else dw.ps_tile_elements(0)
        return dict(desc="u32 exclusive sum scan, n=2^20, values uniform in [0,15], seed 1, " + form,
                    dtype="u32", n=n, bytes=8.0 * n, rbytes=4.0 * n, inputs=dict(x=x), run=run, out=d_out,
                    inclusive=False, kind="u32", tile=tile)
    if name in ("read", "write"):
        # the halves of the copy: 1 GiB only read, 1 GiB only written
        n = wl.N_LARGE_U32
        x = wl.large_u32()
        d_in = dev(x)
        if name == "read":
            sink = torch.zeros(1, dtype=torch.int32, device="cuda")
            run = lambda: dw.ps_read_u32(d_in, sink)  # noqa: E731
            desc = "read-only stream of 2^28 uint32 (1 GiB read)"
        else:
            run = lambda: dw.ps_fill_u32(d_in, 7)  # noqa: E731
            desc = "write-only stream of 2^28 uint32 (1 GiB written)"
        return dict(desc=desc, dtype="u32", n=n, bytes=4.0 * n, rbytes=4.0 * n if name == "read" else 0.0,
                    inputs=dict(x=x), run=run, out=d_in, inclusive=False, kind="copy")
    if name in ("u32x", "u32x-ragged", "u32i", "copy"):
        n = wl.N_RAGGED_U32 if name == "u32x-ragged" else wl.N_LARGE_U32
        x = wl.large_u32()[:n]
        d_in, d_out = dev(x), torch.empty(n, dtype=torch.int32, device="cuda")
        total = torch.zeros(1, dtype=torch.int32, device="cuda")
        if name == "copy":
            desc = "plain copy of 2^28 uint32 (1 GiB read + 1 GiB written)"
            run = lambda: dw.ps_copy_u32(d_in, d_out)  # noqa: E731
        else:
            incl = name == "u32i"
            fn = "ps_scan_inclusive_u32" if incl else "ps_scan_exclusive_u32"
            ws = dw.new_workspace(dw.workspace_bytes(fn, None, None, n, None, None))
            f = getattr(dw, fn)
            run = lambda: f(d_in, d_out, total, workspace=ws)  # noqa: E731
            stats_run = lambda st: dw.ps_scan_lookback_stats("sum", incl, d_in, d_out, st, workspace=ws)  # noqa
            desc = "u32 %s sum scan, n=%s, values uniform in [0,255], seed 2" % (
                "inclusive" if incl else "exclusive", "2^28-12345" if name == "u32x-ragged" else "2^28")
        return dict(desc=desc, dtype="u32", n=n, bytes=8.0 * n, rbytes=4.0 * n, inputs=dict(x=x), run=run,
                    out=d_out, inclusive=(name == "u32i"), kind="copy" if name == "copy" else "u32",
                    stats_run=None if name == "copy" else stats_run,
                    stats_tiles=None if name == "copy" else dw.ps_lookback_tiles(n))
    if name == "u64x":
        n = wl.N_LARGE_U32
        x = wl.large_u32()
        d_in, d_out = dev(x), torch.empty(n, dtype=torch.int64, device="cuda")
        total = torch.zeros(1, dtype=torch.int64, device="cuda")
        ws = dw.new_workspace(dw.workspace_bytes("ps_scan_exclusive_u32_u64", None, None, n, None, None))
        run = lambda: dw.ps_scan_exclusive_u32_u64(d_in, d_out, total, workspace=ws)  # noqa: E731
        return dict(desc="widening u32 -> u64 exclusive sum scan, n=2^28, values uniform in [0,255], seed 2",
                    dtype="u64", n=n, bytes=12.0 * n, rbytes=4.0 * n, inputs=dict(x=x), run=run, out=d_out,
                    inclusive=False, kind="u64")
    if name in ("f32", "f32max"):
        n = wl.N_F32
        x = wl.f32_normal()
        d_in, d_out = dev(x), torch.empty(n, dtype=torch.float32, device="cuda")
        op = "sum" if name == "f32" else "max"
        ws = dw.new_workspace(dw.workspace_bytes("ps_scan", 0, 1, 1, None, None, n, None, None))
        run = lambda: dw.ps_scan(op, True, d_in, d_out, workspace=ws)  # noqa: E731
        stats_run = lambda st: dw.ps_scan_lookback_stats(op, True, d_in, d_out, st, workspace=ws)  # noqa: E731
        return dict(desc="fp32 inclusive %s scan, n=2^27, N(0,1), seed 3" % op, dtype="f32", n=n,
                    bytes=8.0 * n, rbytes=4.0 * n, inputs=dict(x=x), run=run, out=d_out, inclusive=True,
                    kind="f32" + op, stats_run=stats_run, stats_tiles=dw.ps_lookback_tiles(n))
    if name in ("linrec", "linrec-h"):
        # both planes of the scanned pair (16 B per pair), or h = B only (12 B)
        n = wl.N_LINREC
        a, b = wl.linrec_pairs()
        d_a, d_b = dev(a), dev(b)
        d_ob = torch.empty(n, dtype=torch.float32, device="cuda")
        d_oa = torch.empty(n, dtype=torch.float32, device="cuda") if name == "linrec" else None
        ws = dw.new_workspace(dw.workspace_bytes("ps_scan_linrec_f32", None, None, None, None, n, 1, None, None))
        run = lambda: dw.ps_scan_linrec_f32(d_a, d_b, d_ob, out_a=d_oa, inclusive=True,  # noqa: E731
                                            workspace=ws)
        both = name == "linrec"
        stats_run = lambda st: dw.ps_linrec_lookback_stats(d_a, d_b, d_ob, st, out_a=d_oa,  # noqa: E731
                                                           workspace=ws)
        return dict(desc="linear recurrence h[t] = a[t] h[t-1] + b[t] as an inclusive fp32 (a, b) pair scan, "
                         "n=2^27, a ~ U[0.9,1), b ~ N(0,1), seed 6, %s written" % ("A and B" if both else "B = h"),
                    dtype="f32", n=n, bytes=(16.0 if both else 12.0) * n, rbytes=8.0 * n, inputs=dict(a=a, b=b),
                    run=run, out=(d_oa, d_ob), inclusive=True, kind="linrec", stats_run=stats_run,
                    stats_tiles=-(-n // dw.ps_linrec_tile_elements()))
    if name == "segmented":
        values, off = wl.zipf_segments()
        n = values.size
        d_v, d_o = dev(values), dev(off)
        d_out = torch.empty(n, dtype=torch.int32, device="cuda")
        ws = dw.new_workspace(dw.workspace_bytes("ps_segmented_scan_u32", None, n, None, off.size - 1, None, 0, None))
        run = lambda: dw.ps_segmented_scan_u32(d_v, d_o, d_out, inclusive=False, workspace=ws)  # noqa: E731
        stats_run = lambda st: dw.ps_segmented_lookback_stats_u32(d_v, d_o, d_out, st, workspace=ws)  # noqa
        return dict(desc="segmented u32 exclusive sum scan, 2^26 values U[0,1023], 2^16 CSR segments "
                         "(10% empty, one with 25% of the elements, rank-size Zipf(1.2)), seed 5",
                    dtype="u32", n=n, bytes=8.0 * n + 4.0 * off.size, rbytes=4.0 * n + 4.0 * off.size,
                    inputs=dict(x=values, off=off), run=run, out=d_out, inclusive=False, kind="segmented",
                    stats_run=stats_run, stats_tiles=-(-n // dw.ps_segmented_tile_elements()))
    if name in ("compact", "compact-staged"):
        staged = name == "compact-staged"
        rec, flags = wl.compaction_records()
        n = flags.size
        kept = int(flags.sum())
        d_r, d_f = dev(rec), dev(flags)
        d_out = torch.empty_like(d_r)
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        fn = "ps_compact_staged" if staged else "ps_compact"
        ws = dw.new_workspace(dw.workspace_bytes(fn, None, 16, None, n, None, None, None))
        f = getattr(dw, fn)
        run = lambda: f(d_r, d_f, d_out, cnt, workspace=ws)  # noqa: E731
        stats_run = None if staged else (  # noqa: E731
            lambda st: dw.ps_compact_lookback_stats(d_r, d_f, d_out, cnt, st, workspace=ws))
        # staged: flag scan (1 B read, 4 B written) + scatter (1 + 4 + 16 B read)
        # on top of the 16 B written per kept record
        per = (1.0 + 4.0 + 1.0 + 4.0 + 16.0) if staged else 17.0
        return dict(desc="stream compaction of 2^26 16-byte records {u32 id, u32 key, f32 a, f32 b}, "
                         "keep ~ Bernoulli(0.3), seed 4" + (", staged: flag scan then scatter" if staged else ""),
                    dtype="u32", n=n, bytes=per * n + 16.0 * kept + 8.0,
                    rbytes=(22.0 if staged else 17.0) * n, inputs=dict(rec=rec, flags=flags),
                    run=run, out=d_out, count=cnt, inclusive=False, kind="compact",
                    timed_per_step=2 if staged else 1, stats_run=stats_run,
                    stats_tiles=-(-n // dw.ps_compact_tile_records(16)))
    raise SystemExit("unknown workload %r" % name)


def tile_elements(dw, w):
    """Elements (records) per tile of the workload's main kernel."""
    if "tile" in w:
        return w["tile"]
    if w["kind"] == "segmented":
        return dw.ps_segmented_tile_elements()
    if w["kind"] == "compact":
        return dw.ps_compact_tile_records(16)
    if w["kind"] == "copy":
        return None
    if w["kind"] == "linrec":
        return dw.ps_linrec_tile_elements()
    return dw.ps_tile_elements({"f32": 1, "u64": 2}.get(w["dtype"], 0))


def cpu_baseline(w, gpu_out, min_seconds: float):
    """Time the oracle (single-threaded C loop) on the same input; compare."""
    import oracle
    orc = oracle.default()
    kind = w["kind"]
    times = []
    ref = None
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if kind == "u32" or kind == "copy":
            ref = orc.scan_u32(w["inputs"]["x"], "sum", w["inclusive"])[0]
        elif kind == "u64":
            ref = orc.scan_u32_u64(w["inputs"]["x"], w["inclusive"])[0]
        elif kind == "f32sum":
            ref = orc.scan_f32_sum(w["inputs"]["x"], True, want_abs=True)
        elif kind == "f32max":
            ref = orc.scan_f32_minmax(w["inputs"]["x"], "max", True)[0]
        elif kind == "segmented":
            ref = orc.segmented_scan_u32(w["inputs"]["x"], w["inputs"]["off"], False)
        elif kind == "compact":
            ref = orc.compact(w["inputs"]["rec"], w["inputs"]["flags"])
        elif kind == "linrec":
            ref = orc.scan_linrec_f32(np.stack([w["inputs"]["a"], w["inputs"]["b"]], axis=1), True)
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 and time.perf_counter() - t_start >= min_seconds:
            break
    med = statistics.median(times)
    gelems = w["n"] / med / 1e9
    parity = None
    if kind in ("u32", "segmented", "u64"):
        parity = "bit-exact" if np.array_equal(gpu_out, ref) else "MISMATCH"
    elif kind == "f32max":
        parity = "bit-exact" if np.array_equal(gpu_out.view(np.uint32), ref.view(np.uint32)) else "MISMATCH"
    elif kind == "f32sum":
        y, ab, _ = ref
        ok = bool(np.all(np.abs(gpu_out.astype(np.float64) - y) <= 1e-5 * ab))
        parity = "within 1e-5*sum|x|" if ok else "MISMATCH"
    elif kind == "linrec":
        A, B, SA, SB, _ = ref
        ga, gb = gpu_out
        ok = bool(np.all(np.abs(gb.astype(np.float64) - B) <= 1e-5 * SB + 2.0 ** -100))
        if ga is not None:
            ok = ok and bool(np.all(np.abs(ga.astype(np.float64) - A) <= 1e-5 * SA + 2.0 ** -100))
        parity = "within 1e-5*magnitude scan" if ok else "MISMATCH"
    elif kind == "compact":
        out, count = ref
        parity = "bit-exact" if (count == gpu_out[1] and np.array_equal(gpu_out[0][:count], out[:count])) \
            else "MISMATCH"
    sample = "the full %d-element input, %d repetitions (median)" % (w["n"], len(times))
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"value": round(gelems, 4), "unit": "Gelem/s", "cores": 1, "kind": "oracle",
            "sample": sample, "seconds_per_rep": round(med, 4),
            "cores_on_box": os.cpu_count(), "cores_usable": usable,
            "threads_note": "1 of %s host cores (%s usable by this process)" % (os.cpu_count(), usable)}, parity


def flushed_reps(run, reps, flush):
    """R calls, each after a cache flush (outside the timed pair), each timed
    with HIP events on the current stream (the library's); milliseconds."""
    import torch
    times = []
    for _ in range(reps):
        flush.add_(1)  # reads and writes 1 GiB: evicts the L2s and the MALL
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        run()
        end.record()
        end.synchronize()
        times.append(start.elapsed_time(end))
    return {"reps": reps, "median_ms": round(statistics.median(times), 5), "min_ms": round(min(times), 5),
            "max_ms": round(max(times), 5)}


def wall_steps(run, steps, warmup):
    """Milliseconds per call over `steps` calls between two synchronisations."""
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def stream_ceiling(w, steps, reps, flush, scan_ms, scan_flushed_ms):
    """Copy, read and write of 1 GiB in the same process, under the same two
    protocols as the workload, and the workload's ceiling: the copy of the
    same bytes where it reads as many bytes as it writes, else a plain
    stream of its own mix (ps_stream_mix_u32: the bytes both directions
    have moved as a copy, the rest read or written alone; for a read-heavy
    mix also ps_stream_mix_even_u32, the same bytes spread evenly over the
    workgroups, reported beside it), and for the
    recurrence a plain stream of its own shape (two planes read, one or two
    written, ps_stream_planes_f32).  The sum of the read time and the write
    time (`model_ms`) is reported too; it is not a ceiling: a stream that
    both reads and writes runs slower than that sum."""
    import torch

    import device_wide_prefix_chained_amd as dw
    n = 1 << 28
    src = torch.empty(n, dtype=torch.int32, device="cuda").fill_(3)
    dst = torch.empty(n, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    gib = 4.0 * n
    streams = {"copy": lambda: dw.ps_copy_u32(src, dst), "read": lambda: dw.ps_read_u32(src, sink),
               "write": lambda: dw.ps_fill_u32(dst, 7)}
    out = {"bytes_each_way": int(gib)}
    for name, run in streams.items():
        wall = wall_steps(run, steps, 3)
        fl = flushed_reps(run, reps, flush)
        moved = 2 * gib if name == "copy" else gib
        out[name] = {"wall_ms": round(wall, 5), "flushed_median_ms": fl["median_ms"],
                     "gbs_wall": round(moved / (wall * 1e-3) / 1e9, 1),
                     "gbs_flushed": round(moved / (fl["median_ms"] * 1e-3) / 1e9, 1)}
    del src, dst
    if w["kind"] == "linrec":
        # the recurrence's own shape: two planes read, one or two written
        n2 = w["n"]
        pa = torch.empty(n2, dtype=torch.float32, device="cuda").fill_(0.5)
        pb = torch.empty(n2, dtype=torch.float32, device="cuda").fill_(2.0)
        ob = torch.empty(n2, dtype=torch.float32, device="cuda")
        oa = torch.empty(n2, dtype=torch.float32, device="cuda") if w["out"][0] is not None else None
        run = lambda: dw.ps_stream_planes_f32(pa, pb, ob, out_a=oa)  # noqa: E731
        wall = wall_steps(run, steps, 3)
        fl = flushed_reps(run, reps, flush)
        out["planes"] = {"bytes": int(w["bytes"]), "wall_ms": round(wall, 5), "flushed_median_ms": fl["median_ms"],
                         "gbs_wall": round(w["bytes"] / (wall * 1e-3) / 1e9, 1),
                         "gbs_flushed": round(w["bytes"] / (fl["median_ms"] * 1e-3) / 1e9, 1),
                         "frac_wall": round(wall / scan_ms, 4),
                         "frac_flushed": round(fl["median_ms"] / scan_flushed_ms, 4)}
        del pa, pb, ob, oa
    rb = w["rbytes"]
    wb = w["bytes"] - rb
    if rb != wb and w["kind"] != "linrec":
        ni, no = -(-int(rb) // 16) * 4, -(-int(wb) // 16) * 4  # words, whole 16-byte vectors
        mi = torch.empty(ni, dtype=torch.int32, device="cuda").fill_(5)
        mo = torch.empty(no, dtype=torch.int32, device="cuda")
        run = lambda: dw.ps_stream_mix_u32(mi, mo)  # noqa: E731
        wall = wall_steps(run, steps, 3)
        fl = flushed_reps(run, reps, flush)
        moved = 4 * (ni + no)
        out["mix"] = {"bytes_read": 4 * ni, "bytes_written": 4 * no, "wall_ms": round(wall, 5),
                      "flushed_median_ms": fl["median_ms"],
                      "gbs_wall": round(moved / (wall * 1e-3) / 1e9, 1),
                      "gbs_flushed": round(moved / (fl["median_ms"] * 1e-3) / 1e9, 1),
                      "frac_wall": round(wall / scan_ms, 4),
                      "frac_flushed": round(fl["median_ms"] / scan_flushed_ms, 4)}
        if no <= ni:
            # the same mix spread evenly over the workgroups, as a kernel
            # that stores between its loads in every workgroup moves it
            run = lambda: dw.ps_stream_mix_even_u32(mi, mo)  # noqa: E731
            wall = wall_steps(run, steps, 3)
            fl = flushed_reps(run, reps, flush)
            out["mix_even"] = {"wall_ms": round(wall, 5), "flushed_median_ms": fl["median_ms"],
                               "gbs_wall": round(moved / (wall * 1e-3) / 1e9, 1),
                               "gbs_flushed": round(moved / (fl["median_ms"] * 1e-3) / 1e9, 1),
                               "frac_wall": round(wall / scan_ms, 4),
                               "frac_flushed": round(fl["median_ms"] / scan_flushed_ms, 4)}
        del mi, mo
    for proto, key in (("wall", "gbs_wall"), ("flushed", "gbs_flushed")):
        model_ms = (rb / (out["read"][key] * 1e9) + wb / (out["write"][key] * 1e9)) * 1e3
        mine = scan_ms if proto == "wall" else scan_flushed_ms
        out["model_ms_" + proto] = round(model_ms, 5)
        out["frac_of_model_" + proto] = round(model_ms / mine, 4)
    if rb == wb:  # same bytes each way as the copy of the same size
        scale = rb / gib
        out["frac_of_copy_wall"] = round(out["copy"]["wall_ms"] * scale / scan_ms, 4)
        out["frac_of_copy_flushed"] = round(out["copy"]["flushed_median_ms"] * scale / scan_flushed_ms, 4)
    return out


def stream_shapes(steps, rounds=7):
    """The fill, the copy and the read of 1 GiB in every access shape of
    ps_stream_shape (threads per workgroup, 16-byte vectors per thread,
    non-temporal or plain accesses, one-shot or persistent grid) and in the
    library's own ps_fill_u32 / ps_copy_u32 / ps_read_u32.  Each round times every kernel back to back
    like the workload, in a new seeded order (the chip's clock drifts over a
    sweep); per kernel the median over the rounds, and per stream the
    fastest shape next to the library's."""
    import torch

    import device_wide_prefix_chained_amd as dw
    n = 1 << 28
    src = torch.empty(n, dtype=torch.int32, device="cuda").fill_(3)
    dst = torch.empty(n, dtype=torch.int32, device="cuda")
    gib = 4.0 * n
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    kinds = ("write", "copy", "read")
    shapes = [(kind, t, v, x, p) for kind in kinds for t in (64, 128, 256) for v in (4, 8, 16)
              for x in (True, False) for p in (False, True)]
    shapes += [(kind, "library") for kind in kinds]
    library = {"write": lambda: dw.ps_fill_u32(dst, 7), "copy": lambda: dw.ps_copy_u32(src, dst),
               "read": lambda: dw.ps_read_u32(src, sink)}

    def runner(sh):
        if sh[1] == "library":
            return library[sh[0]]
        out, inp = (sink, src) if sh[0] == "read" else (dst, src)
        return lambda: dw.ps_stream_shape(sh[0], out, inp, threads=sh[1], vecs=sh[2], nontemporal=sh[3],
                                          persistent=sh[4], value=7)

    times = {sh: [] for sh in shapes}
    rng = np.random.default_rng(2718)
    for _ in range(rounds):
        for k in rng.permutation(len(shapes)):
            times[shapes[k]].append(wall_steps(runner(shapes[k]), steps, 2))
    del src, dst, sink
    rows = []
    for sh in shapes:
        ms = float(np.median(times[sh]))
        moved = 2 * gib if sh[0] == "copy" else gib
        row = {"stream": sh[0]}
        if sh[1] == "library":
            row["library"] = True
        else:
            row.update(threads=sh[1], vecs=sh[2], nontemporal=sh[3], persistent=sh[4])
        row.update(wall_ms=round(ms, 5), spread_ms=round(float(np.max(times[sh]) - np.min(times[sh])), 5),
                   gbs_wall=round(moved / (ms * 1e-3) / 1e9, 1))
        rows.append(row)
    out = {"bytes_each_way": int(gib), "rounds": rounds, "calls_per_round": steps, "rows": rows}
    for kind in kinds:
        mine = [r for r in rows if r["stream"] == kind and not r.get("library")]
        best = max(mine, key=lambda r: r["gbs_wall"])
        lib_row = next(r for r in rows if r["stream"] == kind and r.get("library"))
        out[kind] = {"best": best, "library_gbs": lib_row["gbs_wall"],
                     "library_frac_of_best": round(lib_row["gbs_wall"] / best["gbs_wall"], 4)}
    return out


def lookback_summary(w, reps, warmup):
    """Run the workload's instrumented kernel (same results, per-tile
    look-back statistics) and summarise the looking tiles: polls and windows
    per look-back, stalled polls, look-back time (the wait after the phase's
    barrier; 100 MHz ticks), and the instrumented call's time."""
    import torch

    import device_wide_prefix_chained_amd as dw
    tiles = w["stats_tiles"]
    st = torch.zeros(dw.STATS_WORDS * tiles, dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        w["stats_run"](st)
    torch.cuda.synchronize()
    rows, times = [], []
    for _ in range(reps):
        st.zero_()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        w["stats_run"](st)
        end.record()
        end.synchronize()
        times.append(start.elapsed_time(end))
        rows.append(st.cpu().numpy().view(np.uint32).reshape(tiles, dw.STATS_WORDS).astype(np.int64))
    a = np.concatenate(rows)
    looking = a[a[:, 0] > 0]
    polls, windows, us, stalls = looking[:, 0], looking[:, 1], looking[:, 2] / 100.0, looking[:, 3]

    def hist(v, top):
        h = {str(k): int(np.sum(v == k)) for k in range(1, top)}
        h["%d+" % top] = int(np.sum(v >= top))
        return h

    pct = lambda q: round(float(np.percentile(us, q)), 2)  # noqa: E731
    # the scan phase of every tile as the control wave saw it: to barrier B,
    # waiting at B, B to barrier A, waiting at A (they add up to the phase)
    ph = a[a[:, 4:8].sum(axis=1) > 0][:, 4:8] / 100.0
    phase = {"phases": int(ph.shape[0]),
             "length_us": {"p10": round(float(np.percentile(ph.sum(axis=1), 10)), 3),
                           "p50": round(float(np.percentile(ph.sum(axis=1), 50)), 3),
                           "p90": round(float(np.percentile(ph.sum(axis=1), 90)), 3),
                           "mean": round(float(ph.sum(axis=1).mean()), 3)}}
    for k, name in enumerate(("control_to_B", "control_waits_at_B", "control_B_to_A", "control_waits_at_A")):
        phase[name + "_us"] = {"p50": round(float(np.percentile(ph[:, k], 50)), 3),
                               "p90": round(float(np.percentile(ph[:, k], 90)), 3),
                               "mean": round(float(ph[:, k].mean()), 3)}
    # a barrier the control wave waits at for at most 20 ns: it came last
    phase["control_last_at_B_pct"] = round(100.0 * float(np.mean(ph[:, 1] <= 0.02)), 1)
    phase["control_last_at_A_pct"] = round(100.0 * float(np.mean(ph[:, 3] <= 0.02)), 1)
    # the timeline of the last call: workgroup starts, first scan phase and
    # end of each workgroup (microseconds from the first workgroup's start)
    r = rows[-1]
    t0 = int(r[:, 11].min())
    rel = lambda v: (v - t0) / 100.0  # noqa: E731
    wgs = {}
    for row in r:
        g = wgs.setdefault(int(row[10]), {"entry": int(row[11]), "first_scan": int(row[8]), "last_scan": int(row[8]),
                                         "end": 0})
        g["first_scan"] = min(g["first_scan"], int(row[8]))
        g["last_scan"] = max(g["last_scan"], int(row[8]))
        if row[12]:
            g["end"] = int(row[12])
    entry = np.array([rel(g["entry"]) for g in wgs.values()])
    first = np.array([rel(g["first_scan"]) for g in wgs.values()])
    last = np.array([rel(g["last_scan"]) for g in wgs.values()])
    end = np.array([rel(g["end"]) for g in wgs.values() if g["end"]])
    q = lambda v: {"min": round(float(v.min()), 2), "p50": round(float(np.median(v)), 2),  # noqa: E731
                   "max": round(float(v.max()), 2)}
    timeline = {"workgroups": len(wgs), "start_us": q(entry), "first_scan_phase_us": q(first),
                "last_scan_phase_us": q(last), "end_us": q(end) if end.size else None,
                "drain_us": q(end - np.array([rel(g["last_scan"]) for g in wgs.values() if g["end"]]))
                if end.size else None}
    arrivals = None
    if w["kind"] == "segmented":
        # the data waves' arrivals at barrier B of each tile's scan phase
        # (word 15, ticks after the control wave's start of the phase)
        w15 = a[:, 15]
        seen = w15 != 0
        first, last = (w15[seen] & 1023) / 100.0, ((w15[seen] >> 10) & 1023) / 100.0
        who = (w15[seen] >> 20) & 15
        ctrl_b = a[seen, 4] / 100.0
        stat = lambda v: {"p50": round(float(np.percentile(v, 50)), 3),  # noqa: E731
                          "p90": round(float(np.percentile(v, 90)), 3), "mean": round(float(v.mean()), 3)}
        arrivals = {"phases": int(seen.sum()), "first_data_wave_us": stat(first),
                    "last_data_wave_us": stat(last), "control_wave_us": stat(ctrl_b),
                    "last_data_wave_index_hist": {str(k): int(np.sum(who == k)) for k in range(16)
                                                  if np.any(who == k)},
                    "control_later_than_last_data_wave_pct": round(100.0 * float(np.mean(ctrl_b > last)), 1)}
    return {"tiles_per_call": tiles, "calls": reps, "looking_tiles_per_call": round(len(looking) / reps, 1),
            "polls_hist": hist(polls, 5), "windows_hist": hist(windows, 4),
            "tiles_with_a_stall_pct": round(100.0 * float(np.mean(stalls > 0)), 2),
            "stalled_polls_per_looking_tile": round(float(stalls.mean()), 3),
            "mean_polls": round(float(polls.mean()), 3),
            "lookback_us": {"p50": pct(50), "p90": pct(90), "p99": pct(99), "max": round(float(us.max()), 2),
                            "mean": round(float(us.mean()), 2)},
            "instrumented_call_ms_median": round(statistics.median(times), 5), "phase": phase,
            "timeline": timeline, "barrier_b_arrivals": arrivals}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="u32x")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum oracle time of the cpu_baseline leg (0 skips it)")
    ap.add_argument("--lookback-stats", type=int, default=0, metavar="R",
                    help="also run the instrumented kernel R times and summarise its look-back "
                         "statistics (u32x, u32i, f32, f32max, segmented, compact, linrec, linrec-h)")
    ap.add_argument("--stream-shapes", action="store_true",
                    help="also time the fill, the copy and the read of 1 GiB in every access shape of "
                         "ps_stream_shape (108 kernels) and in the library's own helpers, 7 rounds")
    ap.add_argument("--flushed-reps", type=int, default=20,
                    help="calls timed one by one after a cache flush, and the same for the "
                         "stream ceilings (0 skips both)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import device_wide_prefix_chained_amd as dw
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dw.lib()

    print("[bench] building workload %s" % args.workload, file=sys.stderr, flush=True)
    w = build_workload(args.workload)
    run = w["run"]
    torch.cuda.synchronize()
    # the warm-up runs instrumented too: the timing events it creates are
    # recycled by the timed steps, which then create none
    dw.ps_kernel_timing(True, every=TIMING_EVERY)
    for _ in range(max(args.warmup, 1)):
        run()
    torch.cuda.synchronize()
    print("[bench] warmup done, timing %d steps" % args.steps, file=sys.stderr, flush=True)

    dw.ps_kernel_timing(True, every=TIMING_EVERY)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms_total, launches = dw.ps_kernel_timing_read()
    dw.ps_kernel_timing(False)

    ms_per_step = elapsed * 1e3 / args.steps
    flushed = ceiling = None
    if args.flushed_reps > 0:
        print("[bench] %d calls after cache flushes" % args.flushed_reps, file=sys.stderr, flush=True)
        flush = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
        flushed = flushed_reps(run, args.flushed_reps, flush)
        print("[bench] stream ceilings (copy, read, write)", file=sys.stderr, flush=True)
        ceiling = stream_ceiling(w, args.steps, args.flushed_reps, flush, ms_per_step, flushed["median_ms"])
        del flush
    shapes = None
    if args.stream_shapes:
        print("[bench] stream shapes", file=sys.stderr, flush=True)
        shapes = stream_shapes(min(args.steps, 20))
    lb = None
    if args.lookback_stats > 0:
        if not w.get("stats_run"):
            raise SystemExit("no instrumented kernel for workload %r" % args.workload)
        print("[bench] look-back statistics, %d calls" % args.lookback_stats, file=sys.stderr, flush=True)
        lb = lookback_summary(w, args.lookback_stats, 3)
    # kernels timed per call: their HIP-event pairs add up to one step
    kernel_ms = kernel_ms_total / max(launches, 1) * w.get("timed_per_step", 1)
    n = w["n"]
    value = n / (ms_per_step * 1e-3) / 1e9
    call_gbs = w["bytes"] / (ms_per_step * 1e-3) / 1e9
    achieved = w["bytes"] / (kernel_ms * 1e-3) / 1e9
    traffic = load_traffic(args.workload, w["bytes"])

    gpu_out = None
    cpu = None
    parity = None
    if args.cpu_seconds > 0:
        if w["kind"] == "compact":
            gpu_out = (w["out"].cpu().numpy().view(np.uint32), int(w["count"].cpu().item()))
        elif w["kind"] == "linrec":
            gpu_out = tuple(None if t is None else t.cpu().numpy() for t in w["out"])
        else:
            o = w["out"].cpu().numpy()
            gpu_out = o.view(np.uint32) if o.dtype == np.int32 else (o.view(np.uint64) if o.dtype == np.int64 else o)
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu, parity = cpu_baseline(w, gpu_out, args.cpu_seconds)

    line = {
        "metric": METRIC if args.workload == "u32x" else "Gelem/s, " + w["desc"],
        "value": round(value, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {"workload": w["desc"], "n": n, "algorithmic_bytes_per_step": w["bytes"],
                   "tile_elements": tile_elements(dw, w)},
        "gbs_per_step": round(call_gbs, 1),
        "pct_hbm_peak_per_step": round(100.0 * call_gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(round(traffic)),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                     "kernel_ms": round(kernel_ms, 5), "timed_launches": launches},
        "cpu_baseline": cpu,
        "parity": parity,
        "timing": {"protocol": "value and ms_per_step: K calls back to back between two synchronisations; "
                               "flushed: calls one by one, caches flushed before each, HIP events",
                   "flushed": flushed},
        "stream_ceiling": ceiling,
    }
    if lb is not None:
        line["lookback_stats"] = lb
    if shapes is not None:
        line["stream_shapes"] = shapes
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
