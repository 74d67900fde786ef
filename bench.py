#!/usr/bin/env python3
"""Throughput of the single-pass device-wide scan on one MI355X.

One step = the exclusive scan of 100,000,007 int32 values (uniform in
[-1000, 1000]) followed by the exclusive scan of 100,000,007 fp32 values
(standard normal), both resident in HBM, both through the C ABI of
libdevscan.so (one look-back kernel launch each). Inputs are synthetic and
seeded (datagen). Prints one JSON line:

  value      whole-job G-elem/s = 2 * n * steps / timed seconds (the K steps
             run back to back)
  roofline   the look-back scan kernel against MI355X peak HBM bandwidth,
             algorithmic bytes 2 * n * 4 per launch:
               frac / achieved  cold: the median of 50 launches of each scan,
                                each after a 1 GiB read that evicts L2 and the
                                memory-side cache (HIP events on the launch
                                stream)
               frac_warm / achieved_warm  the mean launch time over the timed
                                back-to-back steps
  cpu_baseline  the sequential CPU oracle on the host, same inputs (extras
             also carry a second CPU row: a two-pass blocked scan on up to
             16 host threads)
  extras     the same-pattern copy, the three-pass scan, the other
             workloads' scans (one tile, 1M int32, fp32 10M inclusive, int64
             100M), the small ones also replayed from a HIP graph, and
             (unless --no-compact / --no-sort) compaction of 268,435,456
             uint32 keys (ordered, against its read-all / write-half ceiling,
             and both unordered forms), one 8-bit counting-sort pass over
             those keys (with and without values) and MoE alignment of two
             router workloads

Other modes (their own JSON line): --ceiling (the access-pattern table:
read, write, copy and read-all/write-half at 4 to 112 KiB per workgroup,
contiguous and 4 KiB-interleaved, warm and cold), --tile-lds (the pages' LDS
block-scan experiment), --profile-only [--cold] [--pattern ...] (launches
without timing, for rocprofv3).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-compact] [--no-sort]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scan G-elem/s and achieved HBM GB/s (% of peak) at n=100M fp32/int32"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_lookback_scan_100m.json")
KERNEL_SOURCES = ["primitives_device_scan_amd/csrc/tile.hpp", "primitives_device_scan_amd/csrc/device_scan.hpp",
                  "primitives_device_scan_amd/csrc/scan_lookback.hip"]


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


class Evictor:
    """Evicts L2 and the memory-side cache before a cold launch: reads a 1 GiB
    scratch buffer (a reduction, so the lines it leaves behind are clean and
    the next launch writes nothing back). The reduction is queued on the
    current stream, the one the timed launch follows on, with no host wait:
    the next launch starts as soon as the reduction ends, so a start event
    recorded between the two marks the kernel's start and not the host's
    launch path."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        self.sink = torch.zeros((), dtype=torch.float32, device=dev)

    def __call__(self):
        self.sink += self.buf.sum()  # one reduction kernel: reads 1 GiB, writes a few bytes


def cold_times_ms(torch, stream, fn, evict, reps=50):
    """Launch times (ms, HIP events on `stream`) of `reps` launches of fn, each
    right after evict() on the same stream; one launch in flight at a time."""
    out = []
    for _ in range(reps):
        evict()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        out.append(a.elapsed_time(b))
    return out


def measured_traffic(per_launch_alg_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they are absent or were taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = json.load(open(TRAFFIC_FILE))
    if t.get("source_sha") != kernel_source_sha():
        return None
    return t["hbm_bytes_per_launch"]


def check_outputs(x_i, x_f, d_yi, d_yf) -> float:
    """Exits unless the int32 scan equals the oracle's and the fp32 scan is
    within 1e-5 * sum|x| of the fp64 oracle; returns the fp32 max |err|/S."""
    import numpy as np

    import oracle
    if not np.array_equal(d_yi.cpu().numpy(), oracle.scan(x_i, False)):
        log("int32 scan differs from the oracle")
        sys.exit(1)
    y, s = oracle.scan(x_f, False)
    ratio = float(np.max(np.abs(d_yf.cpu().numpy().astype(np.float64) - y) / np.maximum(s, 1e-300)))
    if not ratio <= 1e-5:
        log(f"fp32 scan outside tolerance: max |err|/S = {ratio}")
        sys.exit(1)
    return ratio


def tile_lds_experiment(args):
    """The pages' block-scan table on MI355X: 4,096-element tiles scanned in LDS
    by the work-efficient tree (unpadded, i + i/32, i + i/32 + i/1024) and by
    the double-buffered Hillis-Steele scan, each timed alone and inside the
    three-kernel pipeline, on 10,000,000 fp32 values that are 1.0 except every
    fourth 2.0 (every prefix exact, so the pipeline is checked bit for bit
    before it is timed). GB/s use the pages' 4 * n * 4 bytes for a pipeline."""
    import numpy as np
    import torch

    import datagen
    import primitives_device_scan_amd as ds
    from primitives_device_scan_amd import lds_model

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    L = ds.lib
    n = 10_000_000
    x = torch.from_numpy(datagen.quarter_twos_f32(n)).to(dev)
    y = torch.empty_like(x)
    sums = torch.empty((n + 4095) // 4096, dtype=torch.float32, device=dev)
    i = np.arange(n, dtype=np.int64)
    want = (i + i // 4).astype(np.float32)

    def tile(v):
        st = L.ds_tile_scan(ds.DS_FP32, v, x.data_ptr(), y.data_ptr(), sums.data_ptr(), n, sh)
        if st:
            raise ds.DevscanError(st, "ds_tile_scan")

    def pipe(v):
        st = L.ds_tile_pipeline(ds.DS_FP32, v, x.data_ptr(), y.data_ptr(), n, sh)
        if st:
            raise ds.DevscanError(st, "ds_tile_pipeline")

    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in es:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in es]))

    for name, v in ds.TILE_VARIANTS.items():
        pipe(v)
        torch.cuda.synchronize()
        if not np.array_equal(y.cpu().numpy(), want):
            log(f"pipeline {name} is not exact")
            sys.exit(1)
    if args.profile_only:
        for v in ds.TILE_VARIANTS.values():
            for _ in range(max(1, args.steps)):
                tile(v)
        # the other LDS users, once each: the look-back scan and compaction
        xi = torch.from_numpy(datagen.workload("int32_100m", 10_000_000)).to(dev)
        L.scan_exclusive(ds.DS_INT32, xi.data_ptr(), xi.data_ptr(), xi.numel(), sh)
        cnt = torch.empty(1, dtype=torch.int64, device=dev)
        L.compact_if(ds.DS_INT32, xi.data_ptr(), y.data_ptr(), cnt.data_ptr(), xi.numel(), ds.CMP[">"], 0, sh)
        torch.cuda.synchronize()
        log("profile run done")
        return
    copy_ms = timed(lambda: L.ds_copy(x.data_ptr(), y.data_ptr(), n * 4, sh))
    copy_gbs = 2.0 * n * 4 / (copy_ms * 1e-3) / 1e9
    rows = []
    for name, v in ds.TILE_VARIANTS.items():
        t_ms = timed(lambda: tile(v))
        p_ms = timed(lambda: pipe(v))
        gbs = 4.0 * n * 4 / (p_ms * 1e-3) / 1e9
        row = {"variant": name, "tile_us": round(t_ms * 1e3, 1), "pipeline_us": round(p_ms * 1e3, 1),
               "pipeline_gbs_4n": round(gbs, 1), "pct_of_copy_rate": round(100 * gbs / copy_gbs, 1)}
        if name in lds_model.PADS:
            row["model_requests_per_tile"] = lds_model.tree_requests(lds_model.PADS[name])
            row["model_conflict_cycles_per_tile"] = lds_model.tree_conflict_cycles(pad=lds_model.PADS[name])
        else:
            row["model_requests_per_tile"] = lds_model.hs_requests()
            row["model_conflict_cycles_per_tile"] = 0
        rows.append(row)
    lb_ms = timed(lambda: L.scan_exclusive(ds.DS_FP32, x.data_ptr(), y.data_ptr(), n, sh))
    print(json.dumps({"mode": "tile_lds", "n": n, "dtype": "fp32", "tile": 4096, "threads": 1024,
                      "copy_us": round(copy_ms * 1e3, 1), "copy_gbs": round(copy_gbs, 1), "rows": rows,
                      "lookback_scan_us_same_input": round(lb_ms * 1e3, 1)}), flush=True)


def ceiling_experiment(args):
    """The access-pattern table the scan and the compaction are read against:
    ds_bandwidth_pattern for read / write / copy / read-all-write-half at 4,
    16, 64, 80 and 112 KiB per workgroup, contiguous tiles (the scan's layout) and
    4 KiB chunks at a 32 KiB stride, on 400,000,016 bytes per buffer (the
    100M-element scan's input); plus ds_copy (the scan's own tile) and
    compact_if's read-all-write-half pattern at its 64 KiB tile on 1 GiB.
    Warm: median of 10 back-to-back launches; cold: median of 10 launches each
    after a 1 GiB read."""
    import numpy as np
    import torch

    import primitives_device_scan_amd as ds

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    L = ds.lib
    nbytes = 100_000_007 * 4 // 16 * 16
    a = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    b = torch.zeros_like(a)
    evict = Evictor(torch, dev)

    def warm_ms(fn, reps=10):
        for _ in range(2):
            fn()
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for x, y in es:
            x.record(stream)
            fn()
            y.record(stream)
        torch.cuda.synchronize()
        return float(np.median([x.elapsed_time(y) for x, y in es]))

    rows = []
    for mode, mcode in ds._binding.PATTERNS.items():
        moved = {"read": 1.0, "write": 1.0, "copy": 2.0, "read_half": 1.5, "read_half_held": 1.5, "copy_held": 2.0}[mode]
        for vpt in (1, 4, 16, 20, 28, 32):
            for layout in (0, 1):
                def fn():
                    st = L.ds_bandwidth_pattern(mcode, vpt, layout, a.data_ptr(), b.data_ptr(), nbytes, sh)
                    if st:
                        raise ds.DevscanError(st, "ds_bandwidth_pattern")
                w = warm_ms(fn)
                c = float(np.median(cold_times_ms(torch, stream, fn, evict, reps=10)))
                row = {"mode": mode, "kib_per_workgroup": 4 * vpt,
                       "layout": "contiguous" if layout == 0 else "4KiB_chunks_32KiB_stride",
                       "warm_us": round(w * 1e3, 1), "warm_gbs": round(moved * nbytes / (w * 1e-3) / 1e9, 1),
                       "cold_us": round(c * 1e3, 1), "cold_gbs": round(moved * nbytes / (c * 1e-3) / 1e9, 1)}
                rows.append(row)
                log(f"{mode:9s} {4 * vpt:4d} KiB/WG {row['layout']:24s} warm {row['warm_us']:7.1f} us "
                    f"{row['warm_gbs']:7.1f} GB/s  cold {row['cold_us']:7.1f} us {row['cold_gbs']:7.1f} GB/s")
    cp = lambda: L.ds_copy(a.data_ptr(), b.data_ptr(), nbytes, sh)
    cw, cc = warm_ms(cp), float(np.median(cold_times_ms(torch, stream, cp, evict, reps=10)))
    out = {"mode": "ceiling", "bytes_per_buffer": nbytes, "peak_gbs": PEAK_HBM_GBS, "rows": rows,
           "ds_copy_scan_tile": {"kib_per_workgroup": int(L.ds_tile_elems(ds.DS_INT32, 0)) * 4 // 1024,
                                 "warm_us": round(cw * 1e3, 1), "cold_us": round(cc * 1e3, 1),
                                 "warm_gbs": round(2 * nbytes / (cw * 1e-3) / 1e9, 1),
                                 "cold_gbs": round(2 * nbytes / (cc * 1e-3) / 1e9, 1)}}
    del a, b
    # compaction's own shape: 2^28 uint32 keys, its 64 KiB tile, half written
    nk = 1 << 28
    keys = torch.ones(nk, dtype=torch.int32, device=dev)
    kout = torch.zeros_like(keys)
    cvpt = int(L.ds_tile_elems(ds.DS_UINT32, ds._binding.TILE_OF["compact"])) // 1024
    out["compaction_shape_256m"] = {"kib_per_workgroup": 4 * cvpt, "bytes": int(nk * 6)}
    for mname, mcode in (("held", 4), ("streaming", 3)):
        hf = lambda: L.ds_bandwidth_pattern(mcode, cvpt, 0, keys.data_ptr(), kout.data_ptr(), nk * 4, sh)
        hw, hc = warm_ms(hf), float(np.median(cold_times_ms(torch, stream, hf, evict, reps=10)))
        out["compaction_shape_256m"][mname] = {"warm_us": round(hw * 1e3, 1), "cold_us": round(hc * 1e3, 1)}
    print(json.dumps(out), flush=True)


def profile_pattern(args):
    """--profile-only --pattern MODE:VPT:LAYOUT: --steps launches of one
    ds_bandwidth_pattern case on 400,000,016-byte buffers (each after a 1 GiB
    read with --cold), for counter runs."""
    import torch

    import primitives_device_scan_amd as ds

    mode, vpt, layout = args.pattern.split(":")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = torch.cuda.current_stream().cuda_stream
    nbytes = 100_000_007 * 4 // 16 * 16
    a = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    b = torch.zeros_like(a)
    evict = Evictor(torch, dev) if args.cold else (lambda: None)
    for _ in range(max(1, args.steps)):
        evict()
        st = ds.lib.ds_bandwidth_pattern(ds._binding.PATTERNS[mode], int(vpt), int(layout), a.data_ptr(),
                                         b.data_ptr(), nbytes, sh)
        if st:
            raise ds.DevscanError(st, "ds_bandwidth_pattern")
    torch.cuda.synchronize()
    log(f"profile run done: {args.pattern} x {args.steps}")


def profile_radix(args):
    """--profile-only --workload radix: 8-bit counting-sort passes over the
    compaction keys (268,435,456 uint32), --steps each at shift 0, shift 24,
    shift 0 again (so the order of the legs can be told from the digit),
    then --steps key-value passes at shift 0; for counter runs."""
    import numpy as np
    import torch

    import datagen
    import primitives_device_scan_amd as ds

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = torch.cuda.current_stream().cuda_stream
    nk = datagen.WORKLOADS["compact_256m"][0]
    keys = torch.from_numpy(datagen.workload("compact_256m").view(np.int32)).to(dev)
    vals = torch.from_numpy(datagen.keys_u32(8, nk).view(np.int32)).to(dev)
    kout, vout = torch.empty_like(keys), torch.empty_like(vals)
    for shift in (0, 24, 0):
        for _ in range(max(1, args.steps)):
            st = ds.lib.ds_radix_pass(keys.data_ptr(), kout.data_ptr(), None, None, nk, shift, 8, sh)
            if st:
                raise ds.DevscanError(st, "ds_radix_pass")
    for _ in range(max(1, args.steps)):
        st = ds.lib.ds_radix_pass(keys.data_ptr(), kout.data_ptr(), vals.data_ptr(), vout.data_ptr(), nk, 0, 8, sh)
        if st:
            raise ds.DevscanError(st, "ds_radix_pass kv")
    torch.cuda.synchronize()
    log("profile run done: radix passes")


def profile_compact(args):
    """--profile-only --workload compact: --steps launches each of compact_if
    (ordered), ds_compact_unordered with claims per wave and per workgroup over
    the compaction keys (268,435,456 uint32, keep key < 2^31), then --steps
    copies of 1 GiB (the counters' scale factor); for counter runs."""
    import torch

    import datagen
    import primitives_device_scan_amd as ds

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = torch.cuda.current_stream().cuda_stream
    nk = datagen.WORKLOADS["compact_256m"][0]
    keys = torch.from_numpy(datagen.workload("compact_256m").view("int32")).to(dev)
    out = torch.empty_like(keys)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    evict = Evictor(torch, dev) if args.cold else (lambda: None)
    for _ in range(max(1, args.steps)):
        evict()
        st = ds.lib.compact_if(ds.DS_UINT32, keys.data_ptr(), out.data_ptr(), cnt.data_ptr(), nk, ds.CMP["<"],
                               1 << 31, sh)
        if st:
            raise ds.DevscanError(st, "compact_if")
    for claim in (0, 1):
        for _ in range(max(1, args.steps)):
            evict()
            st = ds.lib.ds_compact_unordered(ds.DS_UINT32, keys.data_ptr(), out.data_ptr(), cnt.data_ptr(), nk,
                                             ds.CMP["<"], 1 << 31, claim, sh)
            if st:
                raise ds.DevscanError(st, "ds_compact_unordered")
    for _ in range(max(1, args.steps)):
        evict()
        st = ds.lib.ds_copy(keys.data_ptr(), out.data_ptr(), nk * 4, sh)
        if st:
            raise ds.DevscanError(st, "ds_copy")
    torch.cuda.synchronize()
    if ds.query_timeout():
        log("a look-back wait gave up")
        sys.exit(1)
    log("profile run done: compaction")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample budget")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--compact", action="store_true", help=argparse.SUPPRESS)  # on by default
    ap.add_argument("--sort", action="store_true", help=argparse.SUPPRESS)     # on by default
    ap.add_argument("--no-compact", action="store_true",
                    help="skip timing compact_if / ds_compact_unordered on 268,435,456 uint32 keys")
    ap.add_argument("--no-sort", action="store_true",
                    help="skip timing the counting-sort pass on 268,435,456 uint32 keys and MoE alignment")
    ap.add_argument("--profile-only", action="store_true",
                    help="inputs, one check, then --steps scans and --steps copies; no timing (for rocprofv3 runs)")
    ap.add_argument("--no-check", action="store_true", help="with --profile-only: skip the oracle check")
    ap.add_argument("--tile-lds", action="store_true",
                    help="the pages' LDS block-scan experiment instead of the main bench (own JSON line)")
    ap.add_argument("--ceiling", action="store_true",
                    help="the access-pattern ceiling table instead of the main bench (own JSON line)")
    ap.add_argument("--cold", action="store_true",
                    help="with --profile-only: a 1 GiB read before every scan launch (the cold protocol)")
    ap.add_argument("--algo", default="default",
                    help="with --profile-only: the ds_scan algorithm the scans use (default, lookback_blocked, ...)")
    ap.add_argument("--workload", default="scan", choices=["scan", "radix", "compact"],
                    help="with --profile-only: radix = counting-sort passes over 2^28 keys (shift 0, then 24, then 0 "
                         "again, --steps each; then --steps key-value passes); compact = compact_if, then "
                         "ds_compact_unordered per wave and per workgroup, then 1 GiB copies, --steps each")
    ap.add_argument("--pattern", default=None,
                    help="with --profile-only: MODE:VPT:LAYOUT of ds_bandwidth_pattern to launch --steps times "
                         "instead of the scans (e.g. write:28:0)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the scan has no multi-GPU path in this library", file=sys.stderr)
        sys.exit(2)

    if args.tile_lds:
        return tile_lds_experiment(args)
    if args.ceiling:
        return ceiling_experiment(args)
    if args.profile_only and args.pattern:
        return profile_pattern(args)
    if args.profile_only and args.workload == "radix":
        return profile_radix(args)
    if args.profile_only and args.workload == "compact":
        return profile_compact(args)

    import numpy as np
    import torch

    import datagen
    import primitives_device_scan_amd as ds

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    L = ds.lib

    n = datagen.WORKLOADS["int32_100m"][0]
    log(f"generating inputs n={n}")
    x_i = datagen.workload("int32_100m")
    x_f = datagen.workload("fp32_100m")
    d_xi = torch.from_numpy(x_i).to(dev)
    d_xf = torch.from_numpy(x_f).to(dev)
    d_yi = torch.empty_like(d_xi)
    d_yf = torch.empty_like(d_xf)
    torch.cuda.synchronize()

    algo = ds.ALGO[args.algo] if args.profile_only else 0  # the timed bench always runs the library default

    def scan_i():
        st = L.ds_scan(ds.DS_INT32, 0, algo, d_xi.data_ptr(), d_yi.data_ptr(), n, sh)
        if st:
            raise ds.DevscanError(st, "scan_exclusive int32")

    def scan_f():
        st = L.ds_scan(ds.DS_FP32, 0, algo, d_xf.data_ptr(), d_yf.data_ptr(), n, sh)
        if st:
            raise ds.DevscanError(st, "scan_exclusive fp32")

    # Check before timing: the oracle on the same bytes.
    scan_i()
    scan_f()
    torch.cuda.synchronize()
    ratio = None
    if args.no_check and args.profile_only:
        log("(oracle check skipped for a counter run)")
    else:
        log("checking against the oracle")
        ratio = check_outputs(x_i, x_f, d_yi, d_yf)
    if ds.query_timeout():
        log("a look-back wait gave up")
        sys.exit(1)

    K, W = args.steps, args.warmup
    if args.profile_only:
        # Scans, then the same-pattern copy of a known size (n*4 bytes read,
        # n*4 bytes written per launch; n*4 rounded down to 16 bytes), whose
        # counters give the scale factor for the scans' FETCH/WRITE_SIZE.
        # --cold: each launch (scans and copies) after a 1 GiB read.
        evict = Evictor(torch, dev) if args.cold else (lambda: None)
        for _ in range(K):
            evict()
            scan_i()
            evict()
            scan_f()
        for _ in range(K):
            evict()
            st = L.ds_copy(d_xi.data_ptr(), d_yi.data_ptr(), n * 4 // 16 * 16, sh)
            if st:
                raise ds.DevscanError(st, "ds_copy")
        torch.cuda.synchronize()
        log("profile run done")
        return

    for _ in range(W):
        scan_i()
        scan_f()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(K):
        ev[k][0].record(stream)
        scan_i()
        ev[k][1].record(stream)
        ev[k][2].record(stream)
        scan_f()
        ev[k][3].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K
    ms_i = [e[0].elapsed_time(e[1]) for e in ev]
    ms_f = [e[2].elapsed_time(e[3]) for e in ev]
    launch_ms = float(np.mean(ms_i + ms_f))
    alg_bytes = 2.0 * n * 4
    achieved = alg_bytes / (launch_ms * 1e-3) / 1e9
    value = 2.0 * n * K / (total_ms * 1e-3) / 1e9
    log(f"timed {K} steps: {ms_step:.4f} ms/step, wall {wall:.3f} s; int32 {np.mean(ms_i)*1e3:.1f} us, "
        f"fp32 {np.mean(ms_f)*1e3:.1f} us per launch")

    extras = {
        "int32_excl_us_mean": round(float(np.mean(ms_i)) * 1e3, 2),
        "fp32_excl_us_mean": round(float(np.mean(ms_f)) * 1e3, 2),
        "int32_excl_us_median": round(float(np.median(ms_i)) * 1e3, 2),
        "fp32_excl_us_median": round(float(np.median(ms_f)) * 1e3, 2),
        "int32_gelem_s": round(n / (float(np.mean(ms_i)) * 1e-3) / 1e9, 2),
        "fp32_gelem_s": round(n / (float(np.mean(ms_f)) * 1e-3) / 1e9, 2),
        "fp32_max_err_over_S": ratio,
        "kernel_source_sha": kernel_source_sha(),
        "context_pages_T4_fp32_100m_gelem_s": 14.9,
    }

    # Same-pattern copy: the practical ceiling (in -> out, 800 MB moved).
    def timed(fn, reps=20, warm=3):
        for _ in range(warm):
            fn()
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in es:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in es]))

    # Cold caches (the headline): 50 launches of each scan, each after a 1 GiB
    # read that evicts L2 and the memory-side cache; medians.
    evict = Evictor(torch, dev)
    cold = {}
    for name, fn in (("int32", scan_i), ("fp32", scan_f)):
        cold[name] = cold_times_ms(torch, stream, fn, evict, reps=50)
        extras[f"{name}_excl_cold_us_median"] = round(float(np.median(cold[name])) * 1e3, 2)
        extras[f"{name}_excl_cold_us_p10_p90"] = [round(float(np.percentile(cold[name], q)) * 1e3, 2) for q in (10, 90)]
    cold_ms = float(np.median(cold["int32"] + cold["fp32"]))

    cpf = lambda: L.ds_copy(d_xi.data_ptr(), d_yi.data_ptr(), n * 4 // 16 * 16, sh)
    cp_ms = timed(cpf)
    cp_cold_ms = float(np.median(cold_times_ms(torch, stream, cpf, evict, reps=20)))
    extras["copy_same_pattern_gbs"] = round(alg_bytes / (cp_ms * 1e-3) / 1e9, 1)
    extras["copy_same_pattern_cold_gbs"] = round(alg_bytes / (cp_cold_ms * 1e-3) / 1e9, 1)
    extras["scan_over_copy"] = round(cp_ms / float(np.median(ms_i)), 4)
    extras["scan_over_copy_cold"] = round(cp_cold_ms / cold_ms, 4)
    # each type's tile held as the scan holds it: no store before the whole tile has arrived
    for name, dcode in (("int32", ds.DS_INT32), ("fp32", ds.DS_FP32)):
        svpt = int(L.ds_scan_tile_elems(dcode, 0, n)) * 4 // 4096
        chf = lambda: L.ds_bandwidth_pattern(5, svpt, 0, d_xi.data_ptr(), d_yi.data_ptr(), n * 4 // 16 * 16, sh)
        ch_cold_ms = float(np.median(cold_times_ms(torch, stream, chf, evict, reps=20)))
        key = "" if name == "int32" else "_fp32_tile"
        extras[f"copy_held{key}_same_pattern_cold_gbs"] = round(alg_bytes / (ch_cold_ms * 1e-3) / 1e9, 1)
        extras[f"{name}_scan_over_copy_held_cold"] = round(ch_cold_ms / float(np.median(cold[name])), 4)
    tp_ms = timed(lambda: L.ds_scan(ds.DS_INT32, 0, ds.ALGO["three_pass"], d_xi.data_ptr(), d_yi.data_ptr(), n, sh))
    extras["three_pass_int32_gelem_s"] = round(n / (tp_ms * 1e-3) / 1e9, 2)
    extras["three_pass_int32_alg_gbs"] = round(alg_bytes / (tp_ms * 1e-3) / 1e9, 1)
    # the blocked tile layout (a measured alternative): both scans, warm and cold
    for name, dcode, dx, dy in (("int32", ds.DS_INT32, d_xi, d_yi), ("fp32", ds.DS_FP32, d_xf, d_yf)):
        bf = lambda: L.ds_scan(dcode, 0, ds.ALGO["lookback_blocked"], dx.data_ptr(), dy.data_ptr(), n, sh)
        extras[f"{name}_excl_blocked_us"] = round(timed(bf) * 1e3, 2)
        extras[f"{name}_excl_blocked_cold_us_median"] = round(
            float(np.median(cold_times_ms(torch, stream, bf, evict, reps=20))) * 1e3, 2)
    # inclusive at the headline size, reusing its buffers
    ii_ms = timed(lambda: L.ds_scan(ds.DS_INT32, 1, 0, d_xi.data_ptr(), d_yi.data_ptr(), n, sh))
    extras["int32_incl_100m_us"] = round(ii_ms * 1e3, 1)
    # both pointers one element past a 16-byte boundary (a tensor slice x[1:])
    mi_ms = timed(lambda: L.ds_scan(ds.DS_INT32, 0, 0, d_xi.data_ptr() + 4, d_yi.data_ptr() + 4, n - 1, sh))
    extras["int32_excl_100m_misaligned_us"] = round(mi_ms * 1e3, 1)
    del d_xf, d_yf

    # the other workloads' configurations, each as its own launch (median of 20)
    def config_time(x_np, dcode, incl):
        dx = torch.from_numpy(x_np).to(dev)
        dy = torch.empty_like(dx)
        ms = timed(lambda: L.ds_scan(dcode, incl, 0, dx.data_ptr(), dy.data_ptr(), x_np.size, sh))
        return ms, dx.numel() * dx.element_size() * 2
    for name, dcode, incl in (("one_tile", ds.DS_INT32, 0), ("mid", ds.DS_INT32, 0), ("mid", ds.DS_INT32, 1),
                              ("fp32_10m", ds.DS_FP32, 1)):
        ms, nbytes = config_time(datagen.workload(name), dcode, incl)
        key = f"{name}_{'incl' if incl else 'excl'}"
        extras[f"{key}_us"] = round(ms * 1e3, 2)
        extras[f"{key}_alg_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    # The same small scans replayed from a HIP graph of 20 launches: the time per
    # launch is then the kernels', not the host's launch path (each replay's
    # result is checked against the eager one first).
    def graph_time(x_np, dcode, incl, calls=20, replays=10):
        dx = torch.from_numpy(x_np).to(dev)
        dy, ref = torch.empty_like(dx), torch.empty_like(dx)
        if L.ds_scan(dcode, incl, 0, dx.data_ptr(), ref.data_ptr(), x_np.size, sh):
            raise ds.DevscanError(1, "ds_scan")
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):  # allocates the capture stream's workspace outside the capture
            L.ds_scan(dcode, incl, 0, dx.data_ptr(), dy.data_ptr(), x_np.size, cap.cuda_stream)
        cap.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for _ in range(calls):
                L.ds_scan(dcode, incl, 0, dx.data_ptr(), dy.data_ptr(), x_np.size, cap.cuda_stream)
        dy.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(dy, ref):
            log("graph replay differs from the eager scan")
            sys.exit(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(replays):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / (calls * replays)
    for name, dcode, incl in (("one_tile", ds.DS_INT32, 0), ("mid", ds.DS_INT32, 0)):
        extras[f"{name}_{'incl' if incl else 'excl'}_graph_us"] = round(
            graph_time(datagen.workload(name), dcode, incl) * 1e3, 2)
    x64 = datagen.uniform_i64(64, n, 40)
    for incl in (0, 1):
        ms, nbytes = config_time(x64, ds.DS_INT64, incl)
        key = f"int64_100m_{'incl' if incl else 'excl'}"
        extras[f"{key}_us"] = round(ms * 1e3, 1)
        extras[f"{key}_alg_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del x64

    if not args.no_compact:
        nk = datagen.WORKLOADS["compact_256m"][0]
        keys = torch.from_numpy(datagen.workload("compact_256m").view(np.int32)).to(dev)
        kout = torch.empty_like(keys)
        cnt = torch.empty(1, dtype=torch.int64, device=dev)
        c_ms = timed(lambda: L.compact_if(ds.DS_UINT32, keys.data_ptr(), kout.data_ptr(), cnt.data_ptr(), nk, 0,
                                          1 << 31, sh), reps=10)
        kept = int(cnt.item())
        cbytes = nk * 4 + kept * 4
        extras["compact_256m_us"] = round(c_ms * 1e3, 1)
        # its ceiling: the same tile and grid reading every key and writing half of them, no scan,
        # held as a single pass must hold it (no store before the whole tile has arrived); and the
        # same bytes streamed (the stored half loaded last and stored at once), for context
        cvpt = int(L.ds_tile_elems(ds.DS_UINT32, ds._binding.TILE_OF["compact"])) * 4 // 4096
        h_ms = timed(lambda: L.ds_bandwidth_pattern(4, cvpt, 0, keys.data_ptr(), kout.data_ptr(), nk * 4, sh), reps=10)
        hs_ms = timed(lambda: L.ds_bandwidth_pattern(3, cvpt, 0, keys.data_ptr(), kout.data_ptr(), nk * 4, sh), reps=10)
        extras["compact_ceiling_256m_us"] = round(h_ms * 1e3, 1)
        extras["compact_over_ceiling"] = round(h_ms / c_ms, 4)
        extras["compact_streaming_256m_us"] = round(hs_ms * 1e3, 1)
        extras["compact_over_streaming"] = round(hs_ms / c_ms, 4)
        extras["compact_256m_gelem_s"] = round(nk / (c_ms * 1e-3) / 1e9, 2)
        extras["compact_256m_alg_gbs"] = round(cbytes / (c_ms * 1e-3) / 1e9, 1)
        # the order-free form: atomic space claims per wave (the pages') and per workgroup
        for claim, code in ds._binding.CLAIM.items():
            u_ms = timed(lambda: L.ds_compact_unordered(ds.DS_UINT32, keys.data_ptr(), kout.data_ptr(),
                                                        cnt.data_ptr(), nk, 0, 1 << 31, code, sh), reps=10)
            if int(cnt.item()) != kept:
                raise SystemExit(f"ds_compact_unordered per {claim}: count {int(cnt.item())} != {kept}")
            extras[f"compact_unordered_per_{claim}_256m_us"] = round(u_ms * 1e3, 1)
        del keys, kout

    if not args.no_sort:
        # one stable 8-bit counting-sort pass (a radix sort's step) over the compaction keys
        nk = datagen.WORKLOADS["compact_256m"][0]
        keys = torch.from_numpy(datagen.workload("compact_256m").view(np.int32)).to(dev)
        vals = torch.from_numpy(datagen.keys_u32(8, nk).view(np.int32)).to(dev)
        kout, vout = torch.empty_like(keys), torch.empty_like(vals)
        # The scatter is bound by VALU issue, so its time follows the clock,
        # which dips for a few ms once back-to-back passes start (470 -> 650 ->
        # 500 us per scatter over the first 15 ms in a kernel trace): each leg
        # is timed after 20 untimed passes.
        for shift in (0, 24):
            r_ms = timed(lambda: L.ds_radix_pass(keys.data_ptr(), kout.data_ptr(), None, None, nk, shift, 8, sh),
                         reps=20, warm=20)
            extras[f"radix_pass_256m_shift{shift}_us"] = round(r_ms * 1e3, 1)
            extras[f"radix_pass_256m_shift{shift}_alg_gbs"] = round(12 * nk / (r_ms * 1e-3) / 1e9, 1)
        rv_ms = timed(lambda: L.ds_radix_pass(keys.data_ptr(), kout.data_ptr(), vals.data_ptr(), vout.data_ptr(), nk,
                                              0, 8, sh), reps=20, warm=20)
        extras["radix_pass_kv_256m_us"] = round(rv_ms * 1e3, 1)
        extras["radix_pass_kv_256m_alg_gbs"] = round(20 * nk / (rv_ms * 1e-3) / 1e9, 1)
        del keys, vals, kout, vout
        for name, (t, k, e, block, _, _) in sorted(datagen.MOE_WORKLOADS.items()):
            ids = torch.from_numpy(datagen.moe_workload(name)).to(dev)
            na = ids.numel()
            cap = na + e * (block - 1)
            counts = torch.empty(e, dtype=torch.int32, device=dev)
            offsets = torch.empty(e + 1, dtype=torch.int32, device=dev)
            srt = torch.empty(cap, dtype=torch.int32, device=dev)
            m_ms = timed(lambda: L.ds_moe_align(ids.data_ptr(), na, e, block, counts.data_ptr(), offsets.data_ptr(),
                                                srt.data_ptr(), cap, sh), reps=20)
            extras[f"moe_align_{name}_us"] = round(m_ms * 1e3, 1)
            # replayed from a HIP graph of 20 calls (checked against the eager call first)
            ref = [t_.clone() for t_ in (counts, offsets, srt)]
            cap_s = torch.cuda.Stream()
            cap_s.wait_stream(stream)
            with torch.cuda.stream(cap_s):  # the capture stream's table and workspace, outside the capture
                L.ds_moe_align(ids.data_ptr(), na, e, block, counts.data_ptr(), offsets.data_ptr(), srt.data_ptr(),
                               cap, cap_s.cuda_stream)
            cap_s.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap_s):
                for _ in range(20):
                    L.ds_moe_align(ids.data_ptr(), na, e, block, counts.data_ptr(), offsets.data_ptr(),
                                   srt.data_ptr(), cap, cap_s.cuda_stream)
            srt.fill_(-9)
            g.replay()
            torch.cuda.synchronize()
            total = int(ref[1][-1].item())
            if not (torch.equal(counts, ref[0]) and torch.equal(offsets, ref[1])
                    and torch.equal(srt[:total], ref[2][:total])):
                log("MoE graph replay differs from the eager call")
                sys.exit(1)
            ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ga.record(stream)
            for _ in range(10):
                g.replay()
            gb.record(stream)
            torch.cuda.synchronize()
            extras[f"moe_align_{name}_graph_us"] = round(ga.elapsed_time(gb) / 200 * 1e3, 2)
            del g

    cpu = None
    if not args.no_cpu:
        log(f"timing the CPU oracle (~{args.cpu_seconds:.0f} s)")
        import oracle
        orc = oracle.default()
        yi = np.empty_like(x_i)
        yf = np.empty(n, dtype=np.float64)
        sf = np.empty(n, dtype=np.float64)
        yi[:] = 0
        yf[:] = 0
        sf[:] = 0
        reps, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and reps < 100:
            c0 = time.perf_counter()
            orc.lib.oracle_scan_u32(x_i.ctypes.data, yi.ctypes.data, n, 0)
            orc.lib.oracle_scan_f32(x_f.ctypes.data, yf.ctypes.data, sf.ctypes.data, n, 0)
            t_cpu += time.perf_counter() - c0
            reps += 1
        cpu = {"value": round(2.0 * n * reps / t_cpu / 1e9, 4), "unit": "G-elem/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} full steps (int32 + fp32 exclusive scans of n={n}), sequential C, "
                         f"{t_cpu:.1f} s on {os.cpu_count()} visible host cores, 1 used",
               "cpu_model": cpu_model()}
        # Second CPU row: the two-pass blocked scan on host threads (reads the
        # input twice), the same full step, median of a few.
        par = oracle.ParallelScan()
        thr = oracle.host_threads()
        yf32 = np.empty_like(x_f)
        par.scan(x_i, False, thr, out=yi)  # untimed: touches the output pages
        par.scan(x_f, False, thr, out=yf32)
        steps_par = []
        while sum(steps_par) < 3.0 and len(steps_par) < 20:
            c0 = time.perf_counter()
            par.scan(x_i, False, thr, out=yi)
            par.scan(x_f, False, thr, out=yf32)
            steps_par.append(time.perf_counter() - c0)
        t_par = float(np.median(steps_par))
        extras["cpu_parallel_baseline"] = {
            "value": round(2.0 * n / t_par / 1e9, 4), "unit": "G-elem/s", "cores": thr,
            "kind": "two-pass blocked scan, one block per thread (pthreads)", "cpu_model": cpu_model(),
            "sample": f"median of {len(steps_par)} full steps (int32 + fp32 exclusive scans of n={n})"}
        del yi, yf, sf, yf32

    traffic = measured_traffic(alg_bytes)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "G-elem/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32+fp32",
        "data": "synthetic",
        "config": {"workload": "exclusive scan, int32 then fp32, n=100,000,007 each (int uniform [-1000,1000], "
                               "fp32 standard normal, seed 4)", "n": n, "algo": "single-pass decoupled look-back",
                   "tile_elems": {"int32": int(L.ds_tile_elems(ds.DS_INT32, 0)),
                                  "fp32": int(L.ds_tile_elems(ds.DS_FP32, 0))},
                   "workgroup": 256},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / (cold_ms * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(alg_bytes / (cold_ms * 1e-3) / 1e9 /
                                                                          PEAK_HBM_GBS, 4),
                     "frac_basis": "cold: median launch time of 50 int32 and 50 fp32 launches, each queued right "
                                   "after a 1 GiB read evicting L2 and the memory-side cache (HIP events on the "
                                   "launch stream, no host wait between the read and the launch)",
                     "launch_us_cold_median": round(cold_ms * 1e3, 2),
                     "achieved_warm": round(achieved, 1), "frac_warm": round(achieved / PEAK_HBM_GBS, 4),
                     "warm_basis": f"mean launch time over the {K} timed back-to-back steps",
                     "launch_us_mean": round(launch_ms * 1e3, 2),
                     "traffic": traffic, "kernel": "lookback_scan_kernel",
                     "alg_bytes_per_launch": int(alg_bytes)},
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
