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
    read; grad_input, grad_offset, grad_mask written (the grad_input clear is
    counted separately)."""
    ho, wo = wl.out_hw
    pg = wl.n * ho * wo * wl.groups
    cg = wl.c // wl.groups
    in_elems = wl.n * wl.h * wl.w * wl.c
    return (2 * in_elems + pg * (cg + 6 * wl.points)) * 4


def traffic_from_profile():
    """HBM bytes per launch measured by rocprofv3 counters, if the committed
    counter summary was taken on the current kernel sources."""
    if not COUNTERS.exists():
        return None
    text = COUNTERS.read_text()
    m_hash = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_val) or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def cpu_baseline(wl, t, images: int):
    import numpy as np
    import oracle

    sl = slice(0, images)
    x = t["x"][sl].double().numpy()
    off = t["offset"][sl].double().numpy()
    m = t["mask"][sl].double().numpy()
    t0 = time.perf_counter()
    oracle.forward(x, off, m, **wl.op_kwargs())
    dt = time.perf_counter() - t0
    samples = wl.samples * images // wl.n
    return {"value": round(samples / dt / 1e9, 6), "unit": "GSamples/s", "cores": 1,
            "kind": "oracle",
            "sample": f"fp64 C oracle, single thread, {images} of {wl.n} images of the same "
                      f"workload ({samples} samples) in {dt:.1f} s"}


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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; multi-GPU runs are not part of it "
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

    value = wl.samples / (ms_per_step * 1e-3) / 1e9
    fwd_bytes = forward_bytes(wl)
    achieved = fwd_bytes / (launch_ms * 1e-3) / 1e9
    traffic = traffic_from_profile()

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
                   "samples_per_step": wl.samples},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "dcn_fwd_kernel",
                     "alg_bytes_per_launch": fwd_bytes,
                     "launch_ms": round(launch_ms, 5)},
    }

    if not args.no_backward and wl.dtype == "f32":
        print("bench: backward", file=sys.stderr, flush=True)
        gx = torch.empty_like(x)
        goff = torch.empty_like(off)
        gmk = torch.empty_like(m)
        nb = max(1, min(args.steps, 20))
        for _ in range(2):
            dcn.dcn_backward(x, off, m, gy, grad_input=gx, grad_offset=goff, grad_mask=gmk, **kw)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(nb):
            dcn.dcn_backward(x, off, m, gy, grad_input=gx, grad_offset=goff, grad_mask=gmk, **kw)
        ev1.record(stream)
        torch.cuda.synchronize()
        bms = ev0.elapsed_time(ev1) / nb
        bbytes = backward_bytes(wl)
        result["backward"] = {"ms_per_call": round(bms, 4),
                              "GSamples_per_s": round(wl.samples / (bms * 1e-3) / 1e9, 3),
                              "alg_GB_per_s": round(bbytes / (bms * 1e-3) / 1e9, 1),
                              "alg_bytes_per_call": bbytes,
                              "note": "includes the grad_input clear"}

    if not args.no_cpu_baseline:
        images = min(wl.n, args.cpu_images or wl.n)
        print(f"bench: CPU oracle on {images} images", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, t, images)

    result["device"] = torch.cuda.get_device_name(dev)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
