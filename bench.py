#!/usr/bin/env python3
"""Throughput of the DCN core forward on one MI355X.

A step is one forward call (offset/mask staging, softmax, sampling locations,
bilinear weights, corner gathers, accumulation, store) over one batch of the
synthetic InternImage-L stage-1 workload: N=32, 96x96, C=160, 10 groups of 16
channels, 3x3 points, fp32, DCNv3 softmax, offsets ~N(0, 1.5).  Inputs are
resident in HBM before the timed region.  Consecutive steps read different
copies of the batch (input sets rotated, together well above the 256 MB
last-level cache), so every step starts from cold caches, as a layer of a
network does; each copy holds the same images in another order.  Before the
timed region the GPU runs the same steps untimed for a fixed wall time, so
that its clocks are steady whatever the step count.  The backward at the same
shape is timed after the forward and reported beside it.

Printed: one JSON line with the throughput (GSamples/s, one sample = one
bilinear sample of a 16-channel group slice), a roofline object for the
forward kernel (algorithmic bytes per launch / the median HIP-event launch
time of the timed steps, against the 8 TB/s HBM peak), the same-run device
copy bandwidth, the host CPU, and the fp64 CPU oracle timed on this host.
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
CSRC = ROOT / "deformable_convolution_vision_dcn_amd" / "csrc"


# The source file of each kernel whose counters the bench reads.
KERNEL_SOURCES = {
    "dcn_fwd_tile_kernel": "dcn_fwd_tile.hip", "dcn_fwd_lane_kernel": "dcn_fwd_lane.hip",
    "dcn_fwd_map_kernel": "dcn_fwd_map.hip", "dcn_fwd_kernel": "dcn_forward.hip",
    "dcn_fused_kernel": "dcn_fused.hip", "dcn_bwd_quad_kernel": "dcn_bwd_quad.hip",
    "dcn_bwd_tile_kernel": "dcn_bwd_tile.hip", "dcn_bwd_kernel": "dcn_backward.hip",
    "dcn_bwd_map_kernel": "dcn_bwd_map.hip",
}


def _code_only(text: str) -> bytes:
    """C/C++ source without its comments and blank space (so that editing a
    comment does not change the hash)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split()).encode()


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code that decides `kernel`'s instructions and launch: its
    own source file, the shared device headers, the host entry points and the
    public header (every library source for a kernel not listed), comments
    left out."""
    h = hashlib.sha256()
    own = KERNEL_SOURCES.get(kernel)
    for f in sorted(CSRC.glob("*")):
        shared = f.suffix in (".hpp", ".h") or f.name == "dcn_api.hip"
        if f.suffix in (".hip", ".hpp", ".h") and (own is None or shared or f.name == own):
            h.update(f.name.encode())
            h.update(_code_only(f.read_text()))
    h.update(_code_only((ROOT / "include" / "dcn.h").read_text()))
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


# Dense matrix-core peaks of MI355X (TFLOP/s) by operand type.
MFMA_PEAK_TFLOPS = {"f32": 157.3, "f16": 2500.0, "bf16": 2500.0}


def generated_cost(wl, cgd: int):
    """(algorithmic bytes, GEMM flops) of one dcn_forward_generated call:
    input once, the guide, the output, the two branches' weights and biases;
    2 flops per multiply-add of the offset and mask GEMM."""
    ho, wo = wl.out_hw
    npix = wl.n * ho * wo
    b = 4 if wl.dtype == "f32" else 2
    cols = wl.groups * wl.points * 3
    nbytes = (wl.n * wl.h * wl.w * wl.c + npix * cgd + npix * wl.c + cols * (cgd + 1)) * b
    return nbytes, 2 * npix * cols * cgd


def projected_cost(wl):
    """(algorithmic bytes, GEMM flops) of one dcn_forward_projected call:
    the core's bytes plus the C x C weight and the bias; 2 flops per
    multiply-add of the projection."""
    ho, wo = wl.out_hw
    npix = wl.n * ho * wo
    b = 4 if wl.dtype == "f32" else 2
    return forward_bytes(wl) + (wl.c * wl.c + wl.c) * b, 2 * npix * wl.c * wl.c


def roofline_of(nbytes: int, flops: int, dtype: str, ms: float) -> dict:
    """The bound (HBM or matrix cores, whichever needs longer at its peak)
    and the achieved rate against it, with both fractions."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS[dtype] * 1e12)
    hbm = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    both = {"hbm_frac": round(hbm / HBM_PEAK_GBS, 4), "mfma_frac": round(tf / MFMA_PEAK_TFLOPS[dtype], 4),
            "hbm_GB_per_s": round(hbm, 1), "mfma_TFLOP_per_s": round(tf, 2),
            "alg_bytes_per_launch": nbytes, "gemm_flops_per_launch": flops}
    if t_mfma > t_hbm:
        return {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
                "frac": round(tf / MFMA_PEAK_TFLOPS[dtype], 4), **both}
    return {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(hbm / HBM_PEAK_GBS, 4), **both}


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


def traced_kernels(fn):
    """Names of the GPU kernels one call of fn() launches, from a torch
    profiler trace of that call (the library's own launches included)."""
    import torch
    from torch.profiler import ProfilerActivity, profile

    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    names = []
    for ev in prof.events():
        if ev.device_type == torch.autograd.DeviceType.CUDA and ev.name not in names:
            names.append(ev.name)
    return names


def short_kernel_name(name: str) -> str:
    """dcn_fwd_tile_kernel out of a demangled template instance name."""
    m = re.search(r"(dcn_\w+?_kernel)", name)
    return m.group(1) if m else name


def counters_path(kernel: str, workload: str) -> pathlib.Path:
    """The committed counter summary of one kernel on one workload."""
    return ROOT / "profiles" / f"{kernel}_{workload}_counters.txt"


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` measured by rocprofv3 counters, if
    the committed counter summary was taken on this workload and the current
    kernel sources."""
    path = counters_path(kernel, workload)
    if not path.exists():
        return None
    text = path.read_text()
    m_hash = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_val) or m_hash.group(1) != kernel_source_hash(kernel):
        return None
    return float(m_val.group(1))


def summarize_counters(root: pathlib.Path, workload: str, kernel: str, command: str) -> str:
    """Turn rocprofv3 --pmc runs of this script into the committed counter
    summary of one kernel: runs "fetch" (FETCH_SIZE) and "write" (WRITE_SIZE)
    of the benchmark, "copy_fetch" and "copy_write" of its --copy-calibration
    mode (each counter scaled by what it reads for a plain device copy of
    known size), and optional runs "l2" (L2 hits and misses), "sq"
    (instruction counts), "wait" (wave-cycles issuing and waiting), "busy"
    (address-unit and L1 busy counters) and "mfma" (matrix-core counters),
    averaged per dispatch of `kernel`."""
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
            raise SystemExit(f"no {counter} rows for {kernel} in {root / run}")
        return [vals[d] for d in sorted(vals)]

    is_kernel = lambda n: short_kernel_name(n) == kernel
    is_copy = lambda n: "copy" in n.lower()
    fetch = per_dispatch("fetch", "FETCH_SIZE", is_kernel)
    write = per_dispatch("write", "WRITE_SIZE", is_kernel)
    cfetch = per_dispatch("copy_fetch", "FETCH_SIZE", is_copy)
    cwrite = per_dispatch("copy_write", "WRITE_SIZE", is_copy)
    copy_bytes = float(1 << 30)
    kib = 1024.0
    f_scale = copy_bytes / (sum(cfetch) / len(cfetch) * kib)
    w_scale = copy_bytes / (sum(cwrite) / len(cwrite) * kib)
    f_bytes = sum(fetch) / len(fetch) * kib * f_scale
    w_bytes = sum(write) / len(write) * kib * w_scale
    from deformable_convolution_vision_dcn_amd import synth

    base, _, mode = workload.partition("_generated") if workload.endswith("_generated") else \
        workload.partition("_projected")
    wl = synth.WORKLOADS[base]
    if workload.endswith("_generated"):
        alg = generated_cost(wl, wl.c)[0]
    elif workload.endswith("_projected"):
        alg = projected_cost(wl)[0]
    else:
        alg = backward_bytes(wl) if "bwd" in kernel else forward_bytes(wl)
    lines = [
        f"# HBM traffic and counters of {kernel}, workload {workload}",
        f"command: {command}",
        f"kernel_source_sha256: {kernel_source_hash(kernel)}",
        f"dispatches_fetch: {len(fetch)}  write: {len(write)}",
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
    for run in ("l2", "sq", "wait", "busy", "mfma"):
        names = set()
        for f in root.glob(f"{run}/**/*counter_collection.csv"):
            for row in csv.DictReader(open(f)):
                names.add(row["Counter_Name"])
        vals = {n: per_dispatch(run, n, is_kernel) for n in sorted(names)}
        for n, v in vals.items():
            lines.append(f"{n}_per_dispatch: {sum(v) / len(v):.4e}")
        if run == "l2" and "TCC_HIT_sum" in vals and "TCC_MISS_sum" in vals:
            h = sum(vals["TCC_HIT_sum"]) / len(vals["TCC_HIT_sum"])
            m = sum(vals["TCC_MISS_sum"]) / len(vals["TCC_MISS_sum"])
            lines.append(f"l2_hit_rate: {h / (h + m):.3f}")
    return "\n".join(lines) + "\n"


# The host CPU share of one GPU on the benchmark machines: worker pools there
# are sized to it, whatever the affinity set shows.
GPU_HOST_SHARE = 16


def host_cpu() -> dict:
    """The host's CPU model, the cores this process may run on, and the
    cores a worker pool here uses (the affinity set, at most one GPU's share
    of the host)."""
    model = "unknown"
    try:
        m = re.search(r"model name\s*:\s*(.*)", pathlib.Path("/proc/cpuinfo").read_text())
        if m:
            model = m.group(1).strip()
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0))
    return {"model": model, "cores_available": avail, "nproc": os.cpu_count(),
            "cores_usable": max(1, min(avail, GPU_HOST_SHARE))}


def cpu_baseline(wl, t, images: int, mode: str = "core", extra=None, guide=None):
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
    host = host_cpu()
    cores = max(1, min(host["cores_usable"], images))

    ex = {k: v.double().numpy() for k, v in (extra or {}).items()}
    gd = guide.cpu()[:images].double().numpy() if guide is not None else None

    def one(i):
        if mode == "generated":
            return oracle.forward_om(x[i:i + 1], gd[i:i + 1], ex["w_offset"], ex["b_offset"], ex["w_mask"],
                                     ex["b_mask"], **kw)
        if mode == "projected":
            return oracle.forward_proj(x[i:i + 1], off[i:i + 1], m[i:i + 1], ex["w_out"], ex["b_out"], **kw)
        return oracle.forward(x[i:i + 1], off[i:i + 1], m[i:i + 1], **kw)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as pool:
        list(pool.map(one, range(images)))
    dt_all = time.perf_counter() - t0
    t0 = time.perf_counter()
    for i in range(images):
        one(i)
    dt_one = time.perf_counter() - t0
    return {"value": round(samples / dt_all / 1e9, 6), "unit": "GSamples/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fp64 C oracle, {images} of {wl.n} images of the same workload "
                      f"({samples} samples), one image per call over {cores} threads, in "
                      f"{dt_all:.2f} s",
            "cpu_model": host["model"], "cores_available": host["cores_available"],
            "single_thread": {"value": round(samples / dt_one / 1e9, 6), "cores": 1,
                              "seconds": round(dt_one, 2)}}


def rotated_sets(tensors, count: int):
    """`count` input sets on the device: the first as given, the others the
    same images in another order (the batch rolled by r images), each in its
    own memory."""
    import torch

    sets = [tensors]
    n = next(iter(tensors.values())).shape[0]
    for r in range(1, count):
        sets.append({k: torch.roll(v, shifts=r % max(n, 1), dims=0).contiguous() for k, v in tensors.items()})
    return sets


def timed_launches(fn, stream, steps: int):
    """Run fn(i) for i < steps back to back on `stream`, a HIP event pair
    around each call: (wall seconds from a synchronised start to a
    synchronised end, sorted per-call milliseconds)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, sorted(a.elapsed_time(b) for a, b in ev)


def dist(times):
    pick = lambda q: times[min(len(times) - 1, int(q * len(times)))]
    return {"median_ms": round(pick(0.5), 5), "mean_ms": round(sum(times) / len(times), 5),
            "min_ms": round(times[0], 5), "p90_ms": round(pick(0.9), 5), "launches": len(times)}


def clock_warmup(fn, seconds: float, at_least: int) -> int:
    """Untimed calls of fn(i) until `seconds` of wall time have passed (and
    at least `at_least` calls), synchronising every 50 calls."""
    import torch

    t0 = time.perf_counter()
    i = 0
    while i < at_least or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def copy_bandwidth(dev, iters: int = 10) -> dict:
    """Device-to-device copy of 1 GiB (torch copy_), per-copy HIP events:
    bytes read plus bytes written over the median copy time."""
    import torch

    a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    stream = torch.cuda.current_stream(dev)
    _, times = timed_launches(lambda i: b.copy_(a), stream, iters)
    med = times[len(times) // 2]
    nbytes = 2 * a.numel() * 4
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_per_copy_read_plus_written": nbytes, "median_ms": round(med, 4),
            "GB_per_s": round(nbytes / (med * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--clock-warmup", type=float, default=2.0,
                    help="seconds of untimed steps before the timed region (clocks settle)")
    ap.add_argument("--workload", default=None, help="named workload (default: stage-1 fp32)")
    ap.add_argument("--mode", choices=["core", "generated", "projected"], default="core",
                    help="core: dcn_forward; generated: offsets and mask generated in the kernel from a guide "
                         "feature (dcn_forward_generated); projected: output_proj fused after the core "
                         "(dcn_forward_projected)")
    ap.add_argument("--sets", type=int, default=None,
                    help="input sets rotated over the steps (default: at least 3 and 1 GiB in all)")
    ap.add_argument("--cpu-images", type=int, default=None,
                    help="images of the batch the CPU oracle runs (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-trace", action="store_true",
                    help="skip the torch-profiler trace that names the kernels (for runs under rocprofv3)")
    ap.add_argument("--remove-center", action="store_true",
                    help="the workload without the kernel's centre point (DCNv4's remove_center)")
    ap.add_argument("--stride", type=int, default=None, help="the workload at this stride (both axes)")
    ap.add_argument("--kernel-size", type=int, default=None,
                    help="the workload with this odd kernel size (pad = dilation * (K - 1) / 2)")
    ap.add_argument("--dilation", type=int, default=None, help="the workload at this dilation (both axes)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--warm-iters", type=int, default=30,
                    help="launches on one input set back to back (warm caches), reported beside")
    ap.add_argument("--flush-iters", type=int, default=20,
                    help="launches each after a 512 MB cache-flushing write, reported beside")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="write the counter summary from rocprofv3 runs under DIR and exit")
    ap.add_argument("--kernel", default=None, help="kernel of --summarize-counters")
    ap.add_argument("--command", default="", help="command recorded in --summarize-counters")
    args = ap.parse_args()

    import deformable_convolution_vision_dcn_amd as dcn
    from deformable_convolution_vision_dcn_amd import synth

    # output extents of the workloads from the library's own host-side check
    synth.set_out_hw(lambda wl: dcn.dcn_check((wl.n, wl.h, wl.w, wl.c), **wl.op_kwargs()))

    if args.summarize_counters:
        text = summarize_counters(pathlib.Path(args.summarize_counters),
                                  args.workload or "stage1_dcnv3_f32", args.kernel or "dcn_fwd_tile_kernel",
                                  args.command)
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

    wl = synth.WORKLOADS[args.workload or synth.HEADLINE]
    if args.remove_center:
        wl = wl.replace(name=wl.name + "_remove_center", remove_center=True)
    if args.stride or args.kernel_size or args.dilation:
        k = args.kernel_size or wl.kernel[0]
        d = args.dilation or wl.dilation[0]
        st = args.stride or wl.stride[0]
        tag = "".join(f"_{n}{v}" for n, v in (("s", args.stride), ("k", args.kernel_size), ("d", args.dilation)) if v)
        wl = wl.replace(name=wl.name + tag, stride=(st, st), kernel=(k, k), dilation=(d, d),
                        pad=(d * (k - 1) // 2, d * (k - 1) // 2))
    dev = torch.device("cuda:0")
    print(f"bench: generating {wl.name}", file=sys.stderr, flush=True)
    mode = args.mode
    if mode != "core":
        args.no_backward = True
    t = synth.make_inputs(wl, with_grad=True)
    base = {k: t[k].to(dev) for k in ("x", "offset", "mask", "grad_out")}
    extra_cpu = {}
    if mode == "generated":
        extra_cpu = synth.make_generation_inputs(wl)
    elif mode == "projected":
        extra_cpu = synth.make_projection_inputs(wl)
    extra = {k: v.to(dev) for k, v in extra_cpu.items()}
    if mode == "generated":
        base = {"x": base["x"], "guide": extra.pop("guide")}
    set_bytes = sum(v.numel() * v.element_size() for k, v in base.items() if k != "grad_out")
    nsets = args.sets or max(3, -(-(1 << 30) // set_bytes))
    sets = rotated_sets(base, nsets)
    kw = wl.op_kwargs()
    y = torch.empty((wl.n, *wl.out_hw, wl.c), dtype=base["x"].dtype, device=dev)
    stream = torch.cuda.current_stream(dev)
    ho_, wo_ = wl.out_hw
    K_ = wl.points

    if mode == "core":
        def fwd(i):
            s_ = sets[i % nsets]
            dcn.dcn_forward(s_["x"], s_["offset"], s_["mask"], out=y, **kw)

        unfused = None
        fwd_bytes, fwd_flops = forward_bytes(wl), 0
    elif mode == "generated":
        def fwd(i):
            s_ = sets[i % nsets]
            dcn.dcn_forward_generated(s_["x"], s_["guide"], extra["w_offset"], extra["b_offset"], extra["w_mask"],
                                      extra["b_mask"], out=y, **kw)

        uoff = torch.empty((wl.n, ho_, wo_, wl.groups, K_, 2), dtype=y.dtype, device=dev)
        umsk = torch.empty((wl.n, ho_, wo_, wl.groups, K_), dtype=y.dtype, device=dev)

        def unfused(i):  # the same step unfused: torch's linear layers, then dcn_forward
            s_ = sets[i % nsets]
            g2 = s_["guide"].view(-1, s_["guide"].shape[3])
            torch.addmm(extra["b_offset"], g2, extra["w_offset"].t(), out=uoff.view(g2.shape[0], -1))
            torch.addmm(extra["b_mask"], g2, extra["w_mask"].t(), out=umsk.view(g2.shape[0], -1))
            dcn.dcn_forward(s_["x"], uoff, umsk, out=y, **kw)

        fwd_bytes, fwd_flops = generated_cost(wl, base["guide"].shape[3])
    else:
        yc = torch.empty_like(y)

        def fwd(i):
            s_ = sets[i % nsets]
            dcn.dcn_forward_projected(s_["x"], s_["offset"], s_["mask"], extra["w_out"], extra["b_out"], out=y,
                                      **kw)

        def unfused(i):  # dcn_forward, then torch's linear layer
            s_ = sets[i % nsets]
            dcn.dcn_forward(s_["x"], s_["offset"], s_["mask"], out=yc, **kw)
            torch.addmm(extra["b_out"], yc.view(-1, wl.c), extra["w_out"].t(), out=y.view(-1, wl.c))

        fwd_bytes, fwd_flops = projected_cost(wl)
    kernels = None
    if not args.no_trace:
        try:
            kernels = [short_kernel_name(k) for k in traced_kernels(lambda: fwd(0))]
        except Exception as e:  # reported, never guessed
            kernels = [f"trace failed: {type(e).__name__}: {e}"]

    print(f"bench: clock warmup {args.clock_warmup} s (at least {args.warmup} steps), "
          f"{nsets} input sets", file=sys.stderr, flush=True)
    warm_calls = clock_warmup(fwd, args.clock_warmup, args.warmup)
    print(f"bench: {args.steps} timed steps", file=sys.stderr, flush=True)
    wall, times = timed_launches(fwd, stream, args.steps)
    ms_per_step = wall * 1e3 / args.steps
    cold = dist(times)
    value = wl.samples / (ms_per_step * 1e-3) / 1e9
    roof = roofline_of(fwd_bytes, fwd_flops, wl.dtype, cold["median_ms"])

    # Beside the graded figure: the same launches on one input set back to
    # back (warm: part of the working set can stay in the 256 MB last-level
    # cache), and each after flushing the caches with 512 MB of other data,
    # once by writing it (its dirty lines are written back during the
    # launch) and once by reading it.
    _, wtimes = timed_launches(lambda i: fwd(0), stream, max(args.warm_iters, 1))
    scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    ftimes, rtimes = [], []
    for _ in range(max(args.flush_iters, 1)):
        scratch.fill_(1.0)
        ftimes += timed_launches(lambda i: fwd(0), stream, 1)[1]
        torch.sum(scratch, dim=0, out=sink)
        rtimes += timed_launches(lambda i: fwd(0), stream, 1)[1]
    del scratch, sink
    ftimes.sort()
    rtimes.sort()
    fwd_kernel = next((k for k in (kernels or []) if k.startswith("dcn_fwd") or k.startswith("dcn_fused")), None)
    wl_label = wl.name if mode == "core" else f"{wl.name}_{mode}"
    traffic = traffic_from_profile(fwd_kernel, wl_label) if fwd_kernel else None
    unfused_stats = None
    if unfused is not None:
        clock_warmup(unfused, 0.5, 5)
        _, utimes = timed_launches(unfused, stream, max(20, min(args.steps, 100)))
        unfused_stats = dist(utimes)

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
        "config": {"workload": wl_label, "n": wl.n, "h": wl.h, "w": wl.w, "c": wl.c,
                   "groups": wl.groups, "kernel": list(wl.kernel), "stride": list(wl.stride),
                   "pad": list(wl.pad), "dilation": list(wl.dilation),
                   "offset_scale": wl.offset_scale, "softmax": wl.softmax,
                   "remove_center": wl.remove_center, "samples_per_step": wl.samples},
        "roofline": {**roof, "traffic": traffic, "kernel": fwd_kernel,
                     "launch_ms": cold["median_ms"],
                     "note": "achieved = algorithmic bytes (or GEMM flops, when the matrix cores bound the "
                             "step) / median per-launch HIP-event time of the timed steps (cold: rotated "
                             "input sets)"},
        "forward_launch": {
            "cold_rotated": cold, "warm_same_set": dist(wtimes), "cold_after_write_flush": dist(ftimes),
            "cold_after_read_flush": dist(rtimes),
            "input_sets": nsets, "input_set_bytes": set_bytes,
            "clock_warmup": {"seconds": args.clock_warmup, "calls": warm_calls},
            "kernels_traced": kernels,
            "unfused_same_step": unfused_stats,
            "note": "cold_rotated: the timed steps, each on another copy of the batch; "
                    "unfused_same_step: the same step as torch linear layers plus dcn_forward; "
                    "warm_same_set: one set back to back; cold_after_write_flush / cold_after_read_flush: "
                    "512 MB written / read before each launch"},
    }

    if not args.no_backward:
        print("bench: backward", file=sys.stderr, flush=True)
        gx = torch.empty_like(base["x"])
        goff = torch.empty_like(base["offset"])
        gmk = torch.empty_like(base["mask"])
        ws_bytes = dcn.backward_workspace_bytes(base["x"], **kw)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        bkw = dict(grad_input=gx, grad_offset=goff, grad_mask=gmk, workspace=ws, **kw)

        def bwd(i):
            s_ = sets[i % nsets]
            dcn.dcn_backward(s_["x"], s_["offset"], s_["mask"], s_["grad_out"], **bkw)

        bkernels = None
        if not args.no_trace:
            try:
                bkernels = [short_kernel_name(k) for k in traced_kernels(lambda: bwd(0))]
            except Exception as e:
                bkernels = [f"trace failed: {type(e).__name__}: {e}"]
        clock_warmup(bwd, 0.5, 2)
        nb = max(1, min(args.steps, 20))
        bwall, btimes = timed_launches(bwd, stream, nb)
        bd = dist(btimes)
        bms = bd["median_ms"]
        bbytes = backward_bytes(wl)
        result["backward"] = {"ms_per_call": bms, "per_call": bd,
                              "GSamples_per_s": round(wl.samples / (bms * 1e-3) / 1e9, 3),
                              "alg_GB_per_s": round(bbytes / (bms * 1e-3) / 1e9, 1),
                              "alg_bytes_per_call": bbytes, "kernels_traced": bkernels,
                              "note": ("median per call on rotated input sets; includes the grad_input clear"
                                       if wl.dtype == "f32" else
                                       "median per call on rotated input sets; includes the fp32 "
                                       "accumulator's clear and rounding")}
    del sets, base
    torch.cuda.empty_cache()
    result["copy_1GiB"] = copy_bandwidth(dev)
    result["host_cpu"] = host_cpu()

    if not args.no_cpu_baseline:
        images = min(wl.n, args.cpu_images or wl.n)
        print(f"bench: CPU oracle on {images} images", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, t, images, mode,
                                              {k: v for k, v in extra_cpu.items() if k != "guide"},
                                              extra_cpu.get("guide"))

    result["device"] = torch.cuda.get_device_name(dev)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
