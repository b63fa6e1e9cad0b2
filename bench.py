#!/usr/bin/env python3
"""Throughput of the DCN core forward on one MI355X.

A step is one forward call (offset/mask staging, softmax, sampling locations,
bilinear weights, corner gathers, accumulation, store) over one batch of the
synthetic InternImage-L stage-1 workload: N=32, 96x96, C=160, 10 groups of 16
channels, 3x3 points, fp32, DCNv3 softmax, offsets ~N(0, 1.5).  Inputs are
resident in HBM before the timed region; steps run back to back on one
stream.  The backward at the same shape is timed after the forward and
reported beside it.

Printed: one JSON line with the throughput (GSamples/s, one sample = one
bilinear sample of a 16-channel group slice), a roofline object for the
forward kernel (algorithmic bytes per launch / HIP-event launch time against
the 8 TB/s HBM peak) and the fp64 CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import pathlib
import re
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "DCN core fwd GSamples/s + achieved HBM GB/s (% peak), InternImage-L stage shapes"
HBM_PEAK_GBS = 8000.0
COUNTERS = ROOT / "profiles" / "dcn_fwd_stage1_dcnv3_f32_counters.txt"
CSRC = ROOT / "deformable_convolution_vision_dcn_amd" / "csrc"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(CSRC.glob("*")):
        if f.suffix in (".hip", ".hpp", ".h"):
            h.update(f.name.encode())
            h.update(f.read_bytes())
    h.update((ROOT / "include" / "dcn.h").read_bytes())
    return h.hexdigest()[:16]


def forward_bytes(wl) -> int:
    """Algorithmic HBM bytes of one forward call: per pixel-group the input
    slice (read once), the output slice, 2K offsets and K mask values."""
    ho, wo = wl.out_hw
    pg = wl.n * ho * wo * wl.groups
    cg = wl.c // wl.groups
    b = {"f32": 4, "f16": 2, "bf16": 2}[wl.dtype]
    in_elems = wl.n * wl.h * wl.w * wl.c
    return (in_elems + pg * (cg + 3 * wl.points)) * b


def backward_bytes(wl) -> int:
    """Algorithmic bytes of one backward call: input, offsets, mask, grad_out
    read; grad_input, grad_offset, grad_mask written, all in the I/O dtype
    (the grad_input clear, and for 16-bit I/O the fp32 accumulator, are the
    implementation's own traffic and not counted)."""
    ho, wo = wl.out_hw
    pg = wl.n * ho * wo * wl.groups
    cg = wl.c // wl.groups
    in_elems = wl.n * wl.h * wl.w * wl.c
    eb = 4 if wl.dtype == "f32" else 2
    return (2 * in_elems + pg * (cg + 6 * wl.points)) * eb


def forward_kernel_name(wl) -> str:
    """Kernel the library runs for this workload's forward (3x3 points,
    stride and dilation 1): the whole-map kernel for output maps smaller than
    a 16x16 tile or that tiles would leave over half empty (the 12x12 stage),
    else the quad tiled kernel for fp32 and the lane-per-pixel-group kernel
    for 16-bit I/O."""
    ho, wo = wl.out_hw
    small = ho * wo < 256 or 2 * ho * wo < ((ho + 15) // 16) * ((wo + 15) // 16) * 256
    if small:
        return "dcn_fwd_map_kernel"
    return "dcn_fwd_tile_kernel" if wl.dtype == "f32" else "dcn_fwd_lane_kernel"


def traffic_from_profile(workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if the committed
    counter summary was taken on this workload and the current kernel
    sources."""
    if not COUNTERS.exists():
        return None
    text = COUNTERS.read_text()
    m_wl = re.search(r"HBM traffic of the forward kernel, workload (\S+)", text)
    m_hash = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_wl and m_hash and m_val) or m_wl.group(1) != workload:
        return None
    if m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def launch_stats(fn, stream, iters: int, flush=None):
    """Per-launch times (ms) of fn() from HIP events on `stream`, one pair of
    events per launch; with `flush`, it runs before each launch, outside the
    events, so every launch starts from cold caches."""
    import torch

    times = []
    for _ in range(iters):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    pick = lambda q: times[min(len(times) - 1, int(q * len(times)))]
    return {"median_ms": round(pick(0.5), 5), "min_ms": round(times[0], 5),
            "p90_ms": round(pick(0.9), 5), "launches": iters}


def summarize_counters(root: pathlib.Path, workload: str) -> str:
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, WRITE_SIZE)
    and two of its --copy-calibration mode into the committed counter
    summary: HBM bytes per forward launch, each counter scaled by what it
    reads for a plain device copy of known size."""
    import csv

    def per_dispatch(run: str, counter: str, match):
        vals = {}
        for f in root.glob(f"{run}/**/*counter_collection.csv"):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] != counter or not match(row["Kernel_Name"]):
                    continue
                d = int(row["Dispatch_Id"])
                vals[d] = vals.get(d, 0.0) + float(row["Counter_Value"])
        if not vals:
            raise SystemExit(f"no {counter} rows in {root / run}")
        return [vals[d] for d in sorted(vals)]

    is_fwd = lambda n: "dcn_fwd" in n
    is_copy = lambda n: "copy" in n.lower()
    fetch = per_dispatch("fetch", "FETCH_SIZE", is_fwd)
    write = per_dispatch("write", "WRITE_SIZE", is_fwd)
    cfetch = per_dispatch("copy_fetch", "FETCH_SIZE", is_copy)
    cwrite = per_dispatch("copy_write", "WRITE_SIZE", is_copy)
    copy_bytes = float(1 << 30)
    kib = 1024.0
    f_scale = copy_bytes / (sum(cfetch) / len(cfetch) * kib)
    w_scale = copy_bytes / (sum(cwrite) / len(cwrite) * kib)
    f_bytes = sum(fetch) / len(fetch) * kib * f_scale
    w_bytes = sum(write) / len(write) * kib * w_scale
    from deformable_convolution_vision_dcn_amd import synth

    alg = forward_bytes(synth.WORKLOADS[workload])
    lines = [
        f"# HBM traffic of the forward kernel, workload {workload}",
        f"kernel_source_sha256: {kernel_source_hash()}",
        f"forward_dispatches_fetch: {len(fetch)}  write: {len(write)}",
        f"FETCH_SIZE_KiB_per_dispatch_raw: {sum(fetch) / len(fetch):.1f}",
        f"WRITE_SIZE_KiB_per_dispatch_raw: {sum(write) / len(write):.1f}",
        f"copy_calibration: 1 GiB device copy, FETCH_SIZE {sum(cfetch) / len(cfetch):.1f} KiB, "
        f"WRITE_SIZE {sum(cwrite) / len(cwrite):.1f} KiB per dispatch",
        f"scale_fetch: {f_scale:.4f}",
        f"scale_write: {w_scale:.4f}",
        f"fetch_bytes_per_launch: {f_bytes:.0f}",
        f"write_bytes_per_launch: {w_bytes:.0f}",
        f"hbm_bytes_per_launch: {f_bytes + w_bytes:.0f}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {(f_bytes + w_bytes) / alg:.3f}",
    ]
    # Optional further runs of this script's timed forward: L2 hits / misses
    # (run "l2") and instruction counters (run "sq"), mean per dispatch.
    for run in ("l2", "sq"):
        names = set()
        for f in root.glob(f"{run}/**/*counter_collection.csv"):
            for row in csv.DictReader(open(f)):
                names.add(row["Counter_Name"])
        vals = {n: per_dispatch(run, n, is_fwd) for n in sorted(names)}
        for n, v in vals.items():
            lines.append(f"{n}_per_dispatch: {sum(v) / len(v):.4e}")
        if run == "l2" and "TCC_HIT_sum" in vals and "TCC_MISS_sum" in vals:
            h = sum(vals["TCC_HIT_sum"]) / len(vals["TCC_HIT_sum"])
            m = sum(vals["TCC_MISS_sum"]) / len(vals["TCC_MISS_sum"])
            lines.append(f"l2_hit_rate: {h / (h + m):.3f}")
    return "\n".join(lines) + "\n"


def cpu_baseline(wl, t, images: int):
    """The fp64 C oracle as it stands, on the first `images` images of the
    same inputs: on all host cores (one image per call, calls spread over a
    thread pool; ctypes releases the GIL, and the oracle keeps no state), and
    on one thread."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    kw = wl.op_kwargs()
    x = t["x"][:images].double().numpy()
    off = t["offset"][:images].double().numpy()
    m = t["mask"][:images].double().numpy()
    samples = wl.samples * images // wl.n
    cores = max(1, min(16, len(os.sched_getaffinity(0)), images))

    def one(i):
        return oracle.forward(x[i:i + 1], off[i:i + 1], m[i:i + 1], **kw)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as pool:
        list(pool.map(one, range(images)))
    dt_all = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.forward(x, off, m, **kw)
    dt_one = time.perf_counter() - t0
    return {"value": round(samples / dt_all / 1e9, 6), "unit": "GSamples/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fp64 C oracle, {images} of {wl.n} images of the same workload "
                      f"({samples} samples), one image per call over {cores} threads, in "
                      f"{dt_all:.2f} s",
            "single_thread": {"value": round(samples / dt_one / 1e9, 6), "cores": 1,
                              "seconds": round(dt_one, 2)}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="named workload (default: stage-1 fp32)")
    ap.add_argument("--cpu-images", type=int, default=None,
                    help="images of the batch the CPU oracle runs (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--remove-center", action="store_true",
                    help="the workload without the kernel's centre point (DCNv4's remove_center)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--cold-iters", type=int, default=50,
                    help="forward launches timed one by one after a 512 MB cache flush")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="write the counter summary from rocprofv3 runs under DIR and exit")
    args = ap.parse_args()

    if args.summarize_counters:
        text = summarize_counters(pathlib.Path(args.summarize_counters),
                                  args.workload or "stage1_dcnv3_f32")
        print(text, end="")
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the DCN core benchmark runs on one GPU; multi-GPU runs are not supported "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        a = torch.ones(1 << 28, device="cuda:0")  # 1 GiB of fp32
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": a.numel() * 4,
                          "copy_calibration_bytes_written": b.numel() * 4, "launches": 5}))
        return 0

    import deformable_convolution_vision_dcn_amd as dcn
    from deformable_convolution_vision_dcn_amd import synth

    wl = synth.WORKLOADS[args.workload or synth.HEADLINE]
    if args.remove_center:
        wl = wl.replace(name=wl.name + "_remove_center", remove_center=True)
    dev = torch.device("cuda:0")
    print(f"bench: generating {wl.name}", file=sys.stderr, flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    x, off, m, gy = (t[k].to(dev) for k in ("x", "offset", "mask", "grad_out"))
    kw = wl.op_kwargs()
    y = torch.empty((wl.n, *wl.out_hw, wl.c), dtype=x.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    print(f"bench: forward warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        dcn.dcn_forward(x, off, m, out=y, **kw)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        dcn.dcn_forward(x, off, m, out=y, **kw)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    launch_ms = ev0.elapsed_time(ev1) / args.steps  # one launch per step at these sizes

    # Per-launch distributions: warm (back to back) and cold (a 512 MB write,
    # twice the MALL and far above the L2s, before every launch).
    fwd = lambda: dcn.dcn_forward(x, off, m, out=y, **kw)
    scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    warm = launch_stats(fwd, stream, max(args.cold_iters, 1))
    cold = launch_stats(fwd, stream, max(args.cold_iters, 1), flush=lambda: scratch.fill_(1.0))
    del scratch

    value = wl.samples / (ms_per_step * 1e-3) / 1e9
    fwd_bytes = forward_bytes(wl)
    achieved = fwd_bytes / (launch_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(wl.name)

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GSamples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded, InternImage-L stage-shaped; no dataset or trained weights)",
        "config": {"workload": wl.name, "n": wl.n, "h": wl.h, "w": wl.w, "c": wl.c,
                   "groups": wl.groups, "kernel": list(wl.kernel), "stride": list(wl.stride),
                   "pad": list(wl.pad), "dilation": list(wl.dilation),
                   "offset_scale": wl.offset_scale, "softmax": wl.softmax,
                   "remove_center": wl.remove_center, "samples_per_step": wl.samples},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": forward_kernel_name(wl),
                     "alg_bytes_per_launch": fwd_bytes,
                     "launch_ms": round(launch_ms, 5)},
        "forward_launch": {
            "warm": warm, "cold": cold,
            "cold_GSamples_per_s": round(wl.samples / (cold["median_ms"] * 1e-3) / 1e9, 3),
            "cold_alg_GB_per_s": round(fwd_bytes / (cold["median_ms"] * 1e-3) / 1e9, 1),
            "note": "cold = 512 MB cache flush before each launch; median of per-launch HIP events"},
    }

    if not args.no_backward:
        print("bench: backward", file=sys.stderr, flush=True)
        gx = torch.empty_like(x)
        goff = torch.empty_like(off)
        gmk = torch.empty_like(m)
        ws_bytes = dcn.backward_workspace_bytes(x, **kw)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device) if ws_bytes else None
        bkw = dict(grad_input=gx, grad_offset=goff, grad_mask=gmk, workspace=ws, **kw)
        nb = max(1, min(args.steps, 20))
        for _ in range(2):
            dcn.dcn_backward(x, off, m, gy, **bkw)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(nb):
            dcn.dcn_backward(x, off, m, gy, **bkw)
        ev1.record(stream)
        torch.cuda.synchronize()
        bms = ev0.elapsed_time(ev1) / nb
        bbytes = backward_bytes(wl)
        result["backward"] = {"ms_per_call": round(bms, 4),
                              "GSamples_per_s": round(wl.samples / (bms * 1e-3) / 1e9, 3),
                              "alg_GB_per_s": round(bbytes / (bms * 1e-3) / 1e9, 1),
                              "alg_bytes_per_call": bbytes,
                              "note": ("includes the grad_input clear" if wl.dtype == "f32" else
                                       "includes the fp32 accumulator's clear and rounding")}

    if not args.no_cpu_baseline:
        images = min(wl.n, args.cpu_images or wl.n)
        print(f"bench: CPU oracle on {images} images", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, t, images)

    result["device"] = torch.cuda.get_device_name(dev)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
