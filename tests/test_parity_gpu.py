"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Bars (the stated parity tolerances of this operator):
  fp32            max |gpu - oracle| <= 1e-4, forward and backward;
  bf16 / fp16     relative error 2e-2, checked elementwise as
                  |gpu - oracle| <= 2e-2 * |oracle| + 1e-3 (an absolute floor
                  for outputs near zero, where a pure ratio is ill-posed).
The oracle sees exactly the values the GPU sees (16-bit inputs widened
exactly) and is not rounded to the I/O dtype.
"""
import math

import numpy as np
import pytest
import torch

import deformable_convolution_vision_dcn_amd as dcn
import oracle
from deformable_convolution_vision_dcn_amd import synth
from deformable_convolution_vision_dcn_amd.synth import Workload, normal, uniform

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ATOL_F32 = 1e-4
RTOL_16, ATOL_16 = 2e-2, 1e-3


def _np(t):
    return t.detach().cpu().double().numpy()


def gate(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert np.array_equal(nan_ref, nan_got), f"{what}: NaN pattern differs"
    g, r = got[~nan_ref], ref[~nan_ref]
    if g.size == 0:
        return
    err = np.abs(g - r)
    if dtype == "f32":
        assert err.max() <= ATOL_F32, f"{what}: max abs error {err.max():.3e} > {ATOL_F32}"
    else:
        bound = RTOL_16 * np.abs(r) + ATOL_16
        worst = int(np.argmax(err - bound))
        assert np.all(err <= bound), (f"{what}: |gpu-ref| {err[worst]:.3e} > bound {bound[worst]:.3e}"
                                      f" at ref {r[worst]:.4e}")


def run_forward(wl, t):
    x, off, m = (t[k].to(DEV) for k in ("x", "offset", "mask"))
    y = dcn.dcn_forward(x, off, m, **wl.op_kwargs())
    torch.cuda.synchronize()
    return y


def oracle_full(wl, t):
    return oracle.forward(_np(t["x"]), _np(t["offset"]), _np(t["mask"]), **wl.op_kwargs())


# --------------------------------------------------------------------------- forward, small

SMALL = [
    Workload("k3_ragged", n=2, h=13, w=11, c=48, groups=3, offset_dist=normal(2.0), seed=11),
    Workload("k3_v4", n=2, h=13, w=11, c=48, groups=3, softmax=False, mask_dist=normal(0.5), seed=12),
    Workload("k3_uniform3", n=3, h=9, w=10, c=32, groups=2, offset_dist=uniform(3.0), seed=13),
    Workload("k3_stride2", n=2, h=15, w=17, c=32, groups=2, stride=(2, 2), pad=(1, 1), seed=14),
    Workload("k3_dil2_pad2", n=1, h=12, w=14, c=64, groups=4, dilation=(2, 2), pad=(2, 2), seed=15),
    Workload("k3_pad0_s1x2", n=2, h=10, w=12, c=16, groups=1, stride=(1, 2), pad=(0, 0), seed=16),
    Workload("k5_generic", n=2, h=9, w=8, c=32, groups=2, kernel=(5, 5), pad=(2, 2), seed=17),
    Workload("k3x5_generic_v4", n=1, h=8, w=11, c=48, groups=3, kernel=(3, 5), pad=(1, 2),
             softmax=False, seed=18),
    Workload("k1_generic", n=2, h=6, w=7, c=32, groups=2, kernel=(1, 1), pad=(0, 0), seed=19),
    Workload("k7_generic_scale1p3", n=1, h=10, w=9, c=16, groups=1, kernel=(7, 7), pad=(3, 3),
             offset_scale=1.3, seed=20),
    Workload("one_pixel", n=1, h=1, w=1, c=16, groups=1, seed=21),
    Workload("wide_many_groups", n=1, h=5, w=37, c=16 * 21, groups=21, seed=22),
    # the centre point removed (8 of the 3x3 points; 14 of a 5x3 grid)
    Workload("rc_k3_v4", n=2, h=13, w=11, c=48, groups=3, softmax=False, mask_dist=normal(0.5),
             remove_center=True, seed=24),
    Workload("rc_k3_v3", n=2, h=12, w=14, c=32, groups=2, offset_dist=uniform(3.0),
             remove_center=True, seed=25),
    Workload("rc_k5x3_stride2", n=1, h=15, w=12, c=32, groups=2, kernel=(5, 3), pad=(2, 1),
             stride=(2, 1), dilation=(1, 2), remove_center=True, seed=26),
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_forward_small(wl, dtype):
    wl = wl.replace(dtype=dtype)
    print(f"forward {wl.name} {dtype}", flush=True)
    t = synth.make_inputs(wl)
    gate(_np(run_forward(wl, t)), oracle_full(wl, t), dtype, f"{wl.name}/{dtype}")


PATH_CASES = [
    Workload("path_ragged", n=2, h=37, w=29, c=48, groups=3, offset_dist=normal(2.0), seed=41),
    Workload("path_far", n=1, h=33, w=35, c=32, groups=2, offset_dist=uniform(5.0), seed=42),
    Workload("path_v4", n=2, h=20, w=17, c=32, groups=2, softmax=False, mask_dist=normal(0.5),
             seed=43),
    Workload("path_pairs", n=2, h=37, w=29, c=96, groups=6, offset_dist=normal(2.5), seed=44),
    # dilation 2: the one-group tiled kernel with its smaller halo (31x31 window)
    Workload("path_dil2", n=2, h=37, w=29, c=48, groups=3, dilation=(2, 2), pad=(2, 2),
             offset_dist=normal(2.0), seed=45),
    # 24 wide, 41 high: 16-bit lane kernel with 24x8 tiles (the last tile row holds one row)
    Workload("path_24wide", n=2, h=41, w=24, c=48, groups=3, offset_dist=uniform(4.0), seed=46),
    # group counts divisible by four (the 16-bit lane kernel's four-group
    # items): ragged 16x16 tiles, the 24-wide tiles with far offsets, and the
    # stage-2 count of 20 groups
    Workload("path_quads", n=2, h=37, w=29, c=128, groups=8, offset_dist=normal(2.5), seed=47),
    Workload("path_quads_v4_24wide", n=2, h=33, w=24, c=64, groups=4, softmax=False,
             mask_dist=normal(0.5), offset_dist=uniform(4.0), seed=48),
    Workload("path_groups20", n=1, h=20, w=18, c=320, groups=20, seed=49),
    # 5x5 points (the lane kernel's 33-pixel-wide windows): four groups, and
    # three with offsets that leave the windows
    Workload("path_k5", n=2, h=37, w=29, c=64, groups=4, kernel=(5, 5), pad=(2, 2), offset_dist=normal(2.0),
             seed=50),
    Workload("path_k5_v4_far", n=1, h=21, w=35, c=48, groups=3, kernel=(5, 5), pad=(2, 2), softmax=False,
             mask_dist=normal(0.5), offset_dist=uniform(8.0), seed=53),
]


@pytest.mark.parametrize("path", ["generic", "tiled", "pair", "lane", "map"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("wl", PATH_CASES, ids=lambda w: w.name)
def test_forward_each_kernel(wl, dtype, path, monkeypatch):
    """Every forward kernel, forced in turn, on shapes spanning several
    tiles with ragged edges and offsets that leave the tile windows."""
    monkeypatch.setenv("DCN_MI355X_FWD_PATH", path)
    wl = wl.replace(dtype=dtype)
    print(f"forward {wl.name} {dtype} path={path}", flush=True)
    t = synth.make_inputs(wl)
    gate(_np(run_forward(wl, t)), oracle_full(wl, t), dtype, f"{wl.name}/{dtype}/{path}")


@pytest.mark.parametrize("groups", [3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_remove_center_every_path(dtype, groups, monkeypatch):
    """With remove_center every forced kernel choice ends in a kernel that
    handles it (the tiled kernels refuse the 8-point rows)."""
    wl = Workload("rc_paths", n=2, h=37, w=29, c=16 * groups, groups=groups, offset_dist=normal(2.0),
                  remove_center=True, dtype=dtype, seed=27)
    t = synth.make_inputs(wl)
    ref = oracle_full(wl, t)
    for path in ["auto", "generic", "tiled", "pair", "lane", "map"]:
        if path == "auto":
            monkeypatch.delenv("DCN_MI355X_FWD_PATH", raising=False)
        else:
            monkeypatch.setenv("DCN_MI355X_FWD_PATH", path)
        print(f"forward rc_paths {dtype} path={path}", flush=True)
        gate(_np(run_forward(wl, t)), ref, dtype, f"rc_paths/{dtype}/{path}")


@pytest.mark.parametrize("groups", [2, 4])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_forward_5x5_remove_center_every_path(dtype, groups, monkeypatch):
    """5x5 points without the centre (24 points, even-length 16-bit mask
    rows) through every forced kernel choice."""
    wl = Workload("rc_k5_paths", n=2, h=24, w=33, c=16 * groups, groups=groups, kernel=(5, 5), pad=(2, 2),
                  offset_dist=normal(2.0), remove_center=True, dtype=dtype, seed=57)
    t = synth.make_inputs(wl)
    ref = oracle_full(wl, t)
    for path in ["auto", "generic", "lane"]:
        if path == "auto":
            monkeypatch.delenv("DCN_MI355X_FWD_PATH", raising=False)
        else:
            monkeypatch.setenv("DCN_MI355X_FWD_PATH", path)
        print(f"forward rc_k5_paths {dtype} G={groups} path={path}", flush=True)
        gate(_np(run_forward(wl, t)), ref, dtype, f"rc_k5_paths/{dtype}/{path}")


# Whole-map kernel: one group per item at the 24x24 stage-3 map (every lane
# busy), four groups per item at 12x12 with a partial last group block (six
# groups), strided and dilated sampling, a wide rectangle, far offsets.
MAP_CASES = [
    Workload("map_24x24", n=3, h=24, w=24, c=160, groups=10, offset_dist=uniform(3.0), seed=51),
    Workload("map_12x12_g6", n=2, h=12, w=12, c=96, groups=6, offset_dist=normal(1.5), seed=52),
    Workload("map_stride2_dil2", n=2, h=20, w=18, c=48, groups=3, stride=(2, 2), dilation=(2, 2),
             pad=(2, 2), seed=53),
    Workload("map_v4_rect", n=2, h=9, w=30, c=64, groups=4, softmax=False, mask_dist=normal(0.5),
             seed=54),
    Workload("map_far", n=1, h=14, w=16, c=32, groups=2, offset_dist=uniform(12.0), seed=55),
    Workload("map_rc_12x12", n=2, h=12, w=12, c=96, groups=6, softmax=False, mask_dist=normal(0.5),
             remove_center=True, seed=56),
    Workload("map_rc_v3_24x24", n=2, h=24, w=24, c=64, groups=4, offset_dist=uniform(3.0),
             remove_center=True, seed=57),
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("wl", MAP_CASES, ids=lambda w: w.name)
def test_forward_map_kernel(wl, dtype, monkeypatch):
    monkeypatch.setenv("DCN_MI355X_FWD_PATH", "map")
    wl = wl.replace(dtype=dtype)
    print(f"forward {wl.name} {dtype} path=map", flush=True)
    t = synth.make_inputs(wl)
    gate(_np(run_forward(wl, t)), oracle_full(wl, t), dtype, f"{wl.name}/{dtype}/map")


# --------------------------------------------------------------------------- forward, full size

def sampled_pixels(wl, count, seed=0):
    ho, wo = wl.out_hw
    total = wl.n * ho * wo
    rng = np.random.default_rng(seed)
    pix = set(rng.integers(0, total, size=min(count, total)).tolist())
    for n in {0, wl.n - 1}:
        for (h, w) in [(0, 0), (0, wo - 1), (ho - 1, 0), (ho - 1, wo - 1), (ho // 2, wo // 2)]:
            pix.add((n * ho + h) * wo + w)
    return np.array(sorted(pix), dtype=np.int64)


def check_sampled(wl, t, y, pixels):
    """Compare y (GPU, full) with the oracle at the given output pixels, one
    image at a time so the oracle only widens that image's tensors."""
    ho, wo = wl.out_hw
    yn = y.view(-1, wl.c)
    per_img = ho * wo
    imgs = pixels // per_img
    for n in np.unique(imgs):
        sel = pixels[imgs == n]
        sl = slice(int(n), int(n) + 1)
        ref = oracle.forward_pixels(_np(t["x"][sl]), _np(t["offset"][sl]), _np(t["mask"][sl]),
                                    sel - n * per_img, **wl.op_kwargs())
        got = _np(yn[torch.from_numpy(sel).to(DEV)])
        gate(got, ref, wl.dtype, f"{wl.name} image {n}")


def check_every_image(wl, t, y):
    """Compare every output element of y (GPU, full batch) with the oracle,
    one image per oracle call (an image's output depends on that image only),
    the calls spread over a thread pool (the oracle keeps no state and ctypes
    releases the GIL)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    kw = wl.op_kwargs()
    x, off, m = t["x"], t["offset"], t["mask"]
    yh = y.cpu()  # one copy to the host; the pool threads touch host memory only

    def one(n):
        sl = slice(n, n + 1)
        ref = oracle.forward(_np(x[sl]), _np(off[sl]), _np(m[sl]), **kw)
        gate(_np(yh[sl]), ref, wl.dtype, f"{wl.name} image {n}")
        return n

    workers = max(1, min(16, len(os.sched_getaffinity(0)), wl.n))
    with ThreadPoolExecutor(workers) as pool:
        done = list(pool.map(one, range(wl.n)))
    assert done == list(range(wl.n))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_named_workload_forward(name):
    """Every named workload at full size, every output element against the
    oracle."""
    wl = synth.WORKLOADS[name]
    print(f"forward {name} (full size, every pixel)", flush=True)
    t = synth.make_inputs(wl, with_grad=False)
    y = run_forward(wl, t)
    assert torch.isfinite(y).all()
    check_every_image(wl, t, y)


def test_forward_multi_chunk():
    """A batch whose input exceeds 2 GiB runs as several launches (chunks of
    whole images); check pixels on both sides of the chunk boundary."""
    wl = Workload("chunked", n=3, h=384, w=384, c=1280, groups=80, offset_dist=normal(1.5), seed=23)
    assert wl.n * wl.h * wl.w * wl.c * 4 > 2 ** 31
    print("forward chunked (3 x 384x384x1280 fp32)", flush=True)
    t = synth.make_inputs(wl, with_grad=False)
    y = run_forward(wl, t)
    check_sampled(wl, t, y, sampled_pixels(wl, 600, seed=1))
    del y, t
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- backward

BWD = [
    Workload("bwd_k3", n=2, h=13, w=11, c=48, groups=3, offset_dist=normal(2.0), seed=31),
    Workload("bwd_k3_v4", n=2, h=12, w=10, c=32, groups=2, softmax=False, mask_dist=normal(0.5), seed=32),
    Workload("bwd_k3_uniform3", n=1, h=9, w=10, c=32, groups=2, offset_dist=uniform(3.0), seed=33),
    Workload("bwd_stride2_dil2", n=2, h=15, w=17, c=32, groups=2, stride=(2, 2), dilation=(2, 2),
             pad=(2, 2), seed=34),
    Workload("bwd_k5_generic", n=1, h=9, w=8, c=32, groups=2, kernel=(5, 5), pad=(2, 2), seed=35),
    Workload("bwd_k3x5_generic_v4", n=1, h=8, w=11, c=16, groups=1, kernel=(3, 5), pad=(1, 2),
             softmax=False, seed=36),
    Workload("bwd_one_pixel", n=1, h=1, w=1, c=16, groups=1, seed=37),
    Workload("bwd_rc_k3_v4", n=2, h=12, w=10, c=32, groups=2, softmax=False, mask_dist=normal(0.5),
             remove_center=True, seed=38),
    Workload("bwd_rc_k3_v3", n=1, h=21, w=19, c=48, groups=3, offset_dist=uniform(3.0),
             remove_center=True, seed=39),
    Workload("bwd_rc_k3x5", n=1, h=9, w=11, c=16, groups=1, kernel=(3, 5), pad=(1, 2),
             remove_center=True, seed=40),
    Workload("bwd_dil2", n=2, h=37, w=29, c=48, groups=3, dilation=(2, 2), pad=(2, 2),
             offset_dist=normal(2.0), seed=41),
]


def run_backward(wl, t):
    x, off, m, gy = (t[k].to(DEV) for k in ("x", "offset", "mask", "grad_out"))
    g = dcn.dcn_backward(x, off, m, gy, **wl.op_kwargs())
    torch.cuda.synchronize()
    return g


def oracle_backward(wl, t):
    return oracle.backward(_np(t["x"]), _np(t["offset"]), _np(t["mask"]), _np(t["grad_out"]),
                           **wl.op_kwargs())


@pytest.mark.parametrize("wl", BWD + [synth.WORKLOADS["hires_dcnv3_f32"], synth.WORKLOADS["tiny_dcnv3_f32"]],
                         ids=lambda w: w.name)
def test_backward(wl):
    print(f"backward {wl.name}", flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    gx, goff, gm = run_backward(wl, t)
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(gx), rx, "f32", f"{wl.name} grad_input")
    gate(_np(goff), roff, "f32", f"{wl.name} grad_offset")
    gate(_np(gm), rm, "f32", f"{wl.name} grad_mask")


BWD_PATH_CASES = [
    Workload("bwdp_ragged", n=2, h=37, w=29, c=48, groups=3, offset_dist=normal(2.0), seed=51),
    Workload("bwdp_far", n=1, h=33, w=35, c=32, groups=2, offset_dist=uniform(5.0), seed=52),
    Workload("bwdp_v4", n=2, h=20, w=17, c=32, groups=2, softmax=False, mask_dist=normal(0.5),
             seed=53),
    Workload("bwdp_pad0", n=1, h=19, w=18, c=16, groups=1, pad=(0, 0), offset_dist=normal(3.0),
             seed=54),
]


# Maps the whole-map backward takes (a 24x24, 16x16 or 12x12 window with its
# border, or a 24x24 one at stride 2): ragged maps smaller than the window,
# padding 0 and 2 (output map smaller or larger than the input), remove_center,
# DCNv4 masks and offsets that leave the map.
BWD_MAP_CASES = [
    Workload("bwdp_map_ragged", n=2, h=20, w=17, c=48, groups=3, offset_dist=uniform(4.0), seed=59),
    Workload("bwdp_map_pad2_v4", n=2, h=10, w=9, c=32, groups=2, pad=(2, 2), softmax=False,
             mask_dist=normal(0.5), offset_dist=normal(2.0), seed=60),
    Workload("bwdp_map16_rc_far", n=1, h=15, w=16, c=32, groups=2, remove_center=True,
             offset_dist=uniform(9.0), seed=61),
    Workload("bwdp_map_pad0", n=2, h=24, w=24, c=16, groups=1, pad=(0, 0), offset_dist=normal(3.0), seed=62),
    Workload("bwdp_map_s2", n=2, h=23, w=21, c=32, groups=2, stride=(2, 2), offset_dist=uniform(4.0), seed=64),
    Workload("bwdp_map_s2_rc_v4", n=1, h=24, w=24, c=48, groups=3, stride=(2, 2), softmax=False,
             mask_dist=normal(0.5), remove_center=True, offset_dist=normal(2.0), seed=65),
]


@pytest.mark.parametrize("path", ["generic", "tiled", "quad", "map"])
@pytest.mark.parametrize("wl", BWD_PATH_CASES + BWD_MAP_CASES + [BWD_PATH_CASES[0].replace(name="bwdp_rc", remove_center=True),
                                BWD_PATH_CASES[1].replace(name="bwdp_dil2_far", dilation=(2, 2), pad=(2, 2)),
                                Workload("bwdp_24wide", n=2, h=41, w=24, c=48, groups=3,
                                         offset_dist=uniform(4.0), seed=55),
                                Workload("bwdp_12x12", n=3, h=12, w=12, c=64, groups=4,
                                         offset_dist=uniform(4.0), seed=56),
                                Workload("bwdp_k5", n=2, h=37, w=29, c=48, groups=3, kernel=(5, 5), pad=(2, 2),
                                         offset_dist=normal(2.0), seed=57),
                                Workload("bwdp_k5_rc_v4_far", n=1, h=33, w=35, c=32, groups=2, kernel=(5, 5),
                                         pad=(2, 2), softmax=False, mask_dist=normal(0.5), remove_center=True,
                                         offset_dist=uniform(6.0), seed=58)],
                         ids=lambda w: w.name)
def test_backward_each_kernel(wl, path, monkeypatch):
    """Every backward kernel, forced in turn, on multi-tile ragged shapes
    whose offsets also leave the tile windows (the global fix-up path), and
    on small maps (the whole-map kernel; a forced kernel that does not take a
    shape falls back to the next)."""
    monkeypatch.setenv("DCN_MI355X_BWD_PATH", path)
    print(f"backward {wl.name} path={path}", flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    gx, goff, gm = run_backward(wl, t)
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(gx), rx, "f32", f"{wl.name}/{path} grad_input")
    gate(_np(goff), roff, "f32", f"{wl.name}/{path} grad_offset")
    gate(_np(gm), rm, "f32", f"{wl.name}/{path} grad_mask")


BWD16 = [
    Workload("bwd16_k3", n=2, h=13, w=11, c=48, groups=3, offset_dist=normal(2.0), seed=61),
    Workload("bwd16_v4", n=2, h=12, w=10, c=32, groups=2, softmax=False, mask_dist=normal(0.5), seed=62),
    Workload("bwd16_ragged_far", n=2, h=37, w=29, c=48, groups=3, offset_dist=uniform(5.0), seed=63),
    Workload("bwd16_pad0", n=1, h=19, w=18, c=16, groups=1, pad=(0, 0), offset_dist=normal(3.0), seed=64),
    Workload("bwd16_one_pixel", n=1, h=1, w=1, c=16, groups=1, seed=65),
    Workload("bwd16_rc_v4", n=2, h=20, w=17, c=32, groups=2, softmax=False, mask_dist=normal(0.5),
             remove_center=True, seed=66),
    Workload("bwd16_rc_far", n=1, h=37, w=29, c=48, groups=3, offset_dist=uniform(5.0),
             remove_center=True, seed=67),
    Workload("bwd16_dil2", n=2, h=30, w=35, c=32, groups=2, dilation=(2, 2), pad=(2, 2),
             offset_dist=normal(2.0), seed=68),
    Workload("bwd16_24wide", n=2, h=24, w=24, c=48, groups=3, offset_dist=uniform(3.0), seed=69),
    Workload("bwd16_12x12", n=3, h=12, w=12, c=64, groups=4, softmax=False, mask_dist=normal(0.5),
             seed=70),
    Workload("bwd16_k5_tiles", n=2, h=37, w=29, c=64, groups=4, kernel=(5, 5), pad=(2, 2),
             offset_dist=normal(2.0), seed=78),
    Workload("bwd16_k5_rc_far", n=1, h=26, w=33, c=48, groups=3, kernel=(5, 5), pad=(2, 2), softmax=False,
             mask_dist=normal(0.5), remove_center=True, offset_dist=uniform(6.0), seed=79),
]


# Shapes beyond 3x3 at stride 1: stride 2 and 5x5 (the tiled quad kernel at
# small sizes) and the untiled kernel's (other strides, dilations and point
# sets), with 16-bit I/O accumulating in fp32.
BWD16_UNTILED = [
    Workload("bwd16_stride2", n=2, h=15, w=17, c=32, groups=2, stride=(2, 2), offset_dist=normal(2.0), seed=71),
    Workload("bwd16_stride2_dil2", n=2, h=15, w=17, c=32, groups=2, stride=(2, 2), dilation=(2, 2),
             pad=(2, 2), seed=72),
    Workload("bwd16_k5", n=1, h=9, w=8, c=32, groups=2, kernel=(5, 5), pad=(2, 2), seed=73),
    Workload("bwd16_k3x5_v4", n=1, h=8, w=11, c=48, groups=3, kernel=(3, 5), pad=(1, 2), softmax=False,
             mask_dist=normal(0.5), seed=74),
    Workload("bwd16_rc_k5x3_s2", n=1, h=15, w=12, c=32, groups=2, kernel=(5, 3), pad=(2, 1), stride=(2, 1),
             dilation=(1, 2), remove_center=True, seed=75),
    Workload("bwd16_k1", n=2, h=6, w=7, c=32, groups=2, kernel=(1, 1), pad=(0, 0), offset_dist=uniform(3.0),
             seed=76),
    Workload("bwd16_dil_1x2", n=1, h=19, w=23, c=16, groups=1, dilation=(1, 2), pad=(1, 2),
             offset_dist=uniform(5.0), seed=77),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("wl", BWD16_UNTILED, ids=lambda w: w.name)
def test_backward_16bit_untiled_shapes(wl, dtype):
    """16-bit backward on shapes outside the tiled kernel's (stride 2, 5x5,
    3x5, 1x1, dilation on one axis, remove_center on a 5x3 grid), against the
    oracle on the 16-bit gate."""
    wl = wl.replace(dtype=dtype)
    print(f"backward {wl.name} {dtype}", flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    gx, goff, gm = run_backward(wl, t)
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(gx), rx, dtype, f"{wl.name}/{dtype} grad_input")
    gate(_np(goff), roff, dtype, f"{wl.name}/{dtype} grad_offset")
    gate(_np(gm), rm, dtype, f"{wl.name}/{dtype} grad_mask")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("wl", [BWD16[2], BWD16[5], BWD16[7]], ids=lambda w: w.name)
def test_backward_16bit_forced_untiled(wl, dtype, monkeypatch):
    """The untiled 16-bit backward forced on shapes the tiled kernel takes by
    default (ragged far offsets, remove_center, dilation 2)."""
    monkeypatch.setenv("DCN_MI355X_BWD_PATH", "generic")
    wl = wl.replace(dtype=dtype)
    print(f"backward {wl.name} {dtype} path=generic", flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    gx, goff, gm = run_backward(wl, t)
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(gx), rx, dtype, f"{wl.name}/{dtype}/generic grad_input")
    gate(_np(goff), roff, dtype, f"{wl.name}/{dtype}/generic grad_offset")
    gate(_np(gm), rm, dtype, f"{wl.name}/{dtype}/generic grad_mask")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("wl", BWD16, ids=lambda w: w.name)
def test_backward_16bit(wl, dtype):
    """16-bit backward (3x3 with or without the centre, stride 1, dilation 1
    or 2) against the oracle on the same 16-bit inputs, with the 16-bit gate
    on all three gradients."""
    wl = wl.replace(dtype=dtype)
    print(f"backward {wl.name} {dtype}", flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    gx, goff, gm = run_backward(wl, t)
    assert gx.dtype == t["x"].dtype and goff.dtype == gx.dtype and gm.dtype == gx.dtype
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(gx), rx, dtype, f"{wl.name}/{dtype} grad_input")
    gate(_np(goff), roff, dtype, f"{wl.name}/{dtype} grad_offset")
    gate(_np(gm), rm, dtype, f"{wl.name}/{dtype} grad_mask")


def test_backward_adjoint_at_stage1_size():
    """At the stage-1 size (too big for a quick full oracle backward) the
    grad_input is checked by the adjoint identity <F(x), g> = <x, F^T g>,
    which holds at any size, and grad_offset / grad_mask on sampled rows."""
    wl = synth.WORKLOADS["stage1_dcnv3_f32"].replace(backward=True)
    print("backward stage1 (adjoint)", flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    y = run_forward(wl, t)
    gx, goff, gm = run_backward(wl, t)
    x, gy = t["x"].to(DEV).double(), t["grad_out"].to(DEV).double()
    terms = y.double() * gy
    lhs = float(terms.sum())
    rhs = float((x * gx.double()).sum())
    # fp32 rounding of each term is ~1e-7 relative; bound by the sum of |terms|
    assert abs(lhs - rhs) <= 1e-6 * float(terms.abs().sum()), (lhs, rhs)
    # rows of image 0 and the last image, checked against the oracle on a
    # one-image slice
    for n in (0, wl.n - 1):
        sl = slice(n, n + 1)
        sub = {k: v[sl] for k, v in t.items()}
        w1 = wl.replace(n=1)
        rx, roff, rm = oracle_backward(w1, sub)
        # grad_input of image n depends only on image n
        gate(_np(gx[sl]), rx, "f32", f"stage1 grad_input image {n}")
        gate(_np(goff[sl]), roff, "f32", f"stage1 grad_offset image {n}")
        gate(_np(gm[sl]), rm, "f32", f"stage1 grad_mask image {n}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_backward_16bit_at_stage1_size(dtype):
    """16-bit backward at the stage-1 size: grad_input by the adjoint identity
    and all three gradients of the first and last image against the oracle.
    The adjoint sides differ by the 16-bit rounding of y and grad_input (at
    most half an ulp, 2^-9 relative for bf16, of each) plus fp32 sums, so the
    bound is 2^-8 of the sum of both sides' absolute terms."""
    wl = synth.WORKLOADS["stage1_dcnv3_f32"].replace(backward=True, dtype=dtype)
    print(f"backward stage1 {dtype} (adjoint)", flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    y = run_forward(wl, t)
    gx, goff, gm = run_backward(wl, t)
    x, gy = t["x"].to(DEV).double(), t["grad_out"].to(DEV).double()
    lhs_t = y.double() * gy
    rhs_t = x * gx.double()
    bound = 2.0 ** -8 * float(lhs_t.abs().sum() + rhs_t.abs().sum())
    assert abs(float(lhs_t.sum()) - float(rhs_t.sum())) <= bound
    for n in (0, wl.n - 1):
        sl = slice(n, n + 1)
        sub = {k: v[sl] for k, v in t.items()}
        rx, roff, rm = oracle_backward(wl.replace(n=1), sub)
        gate(_np(gx[sl]), rx, dtype, f"stage1/{dtype} grad_input image {n}")
        gate(_np(goff[sl]), roff, dtype, f"stage1/{dtype} grad_offset image {n}")
        gate(_np(gm[sl]), rm, dtype, f"stage1/{dtype} grad_mask image {n}")


def test_backward_16bit_reuses_a_workspace():
    """Two 16-bit backward calls in a row through one caller workspace (left
    dirty by the first) give the results of calls with fresh workspaces."""
    wl = BWD16[2].replace(dtype="bf16")
    t = synth.make_inputs(wl, with_grad=True)
    x, off, m, gy = (t[k].to(DEV) for k in ("x", "offset", "mask", "grad_out"))
    need = dcn.backward_workspace_bytes(x, **wl.op_kwargs())
    assert need == x.numel() * 4
    ws = torch.full((need + 64,), 0x7f, dtype=torch.uint8, device=DEV)
    ref = [_np(g) for g in dcn.dcn_backward(x, off, m, gy, **wl.op_kwargs())]
    small = wl.replace(n=1)
    ref1 = [_np(g) for g in dcn.dcn_backward(x[:1], off[:1], m[:1], gy[:1], **small.op_kwargs())]
    for _ in range(2):
        got = [_np(g) for g in dcn.dcn_backward(x, off, m, gy, workspace=ws, **wl.op_kwargs())]
        got1 = [_np(g) for g in dcn.dcn_backward(x[:1], off[:1], m[:1], gy[:1], workspace=ws,
                                                  **small.op_kwargs())]
        torch.cuda.synchronize()
        for a, b in zip(got + got1, ref + ref1):
            # fp32 atomics make grad_input's rounding order vary: 1 ulp of bf16 at most
            np.testing.assert_allclose(a, b, rtol=2.0 ** -7, atol=1e-6)
    with pytest.raises(dcn.DCNError, match="WORKSPACE"):
        dcn.dcn_backward(x, off, m, gy, workspace=ws[: need - 16], **wl.op_kwargs())


def test_backward_16bit_multi_chunk():
    """A bf16 batch whose fp32 grad_input accumulator exceeds 2 GiB runs as
    chunks of two images through one workspace; an image of the first and of
    the second chunk gets the gradients of a one-image call (grad_offset and
    grad_mask bit for bit, grad_input within one bf16 ulp and the fp32
    rounding of its partial sums: the order of its fp32 atomics may
    differ)."""
    wl = Workload("chunked_bwd16", n=3, h=384, w=384, c=1280, groups=80, dtype="bf16",
                  offset_dist=normal(1.5), seed=28)
    img32 = wl.h * wl.w * wl.c * 4
    assert wl.n * img32 > 2 ** 31 and 2 * img32 < 2 ** 31
    print("backward chunked bf16 (3 x 384x384x1280)", flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    x, off, m, gy = (t[k].to(DEV) for k in ("x", "offset", "mask", "grad_out"))
    del t
    kw = wl.op_kwargs()
    assert dcn.backward_workspace_bytes(x, **kw) == 2 * img32
    batch = dcn.dcn_backward(x, off, m, gy, **kw)
    for n in (1, 2):
        sl = slice(n, n + 1)
        one = dcn.dcn_backward(x[sl], off[sl], m[sl], gy[sl], **kw)
        torch.cuda.synchronize()
        assert torch.equal(batch[1][sl], one[1]), f"grad_offset of image {n}"
        assert torch.equal(batch[2][sl], one[2]), f"grad_mask of image {n}"
        a, b = batch[0][sl].float(), one[0].float()
        # one bf16 ulp of the value, plus the fp32 rounding of partial sums of
        # magnitude O(10) where the total nearly cancels
        d = (a - b).abs()
        bad = d > 2.0 ** -7 * b.abs() + 1e-5
        assert not bool(bad.any()), (f"grad_input of image {n}: {int(bad.sum())} elements, max diff "
                                     f"{float(d.max()):.3e}, max |ref| {float(b.abs().max()):.3e}, "
                                     f"differing {int((d > 0).sum())} of {d.numel()}")
        del one
    del batch, x, off, m, gy
    torch.cuda.empty_cache()


def test_autograd_function_matches_backward():
    wl = BWD[0]
    t = synth.make_inputs(wl, with_grad=True)
    x, off, m, gy = (t[k].to(DEV).requires_grad_(k != "grad_out") for k in ("x", "offset", "mask", "grad_out"))
    y = dcn.dcn_core(x, off, m, **wl.op_kwargs())
    gx, goff, gm = torch.autograd.grad(y, (x, off, m), grad_outputs=gy)
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(gx), rx, "f32", "autograd grad_input")
    gate(_np(goff), roff, "f32", "autograd grad_offset")
    gate(_np(gm), rm, "f32", "autograd grad_mask")


@pytest.mark.parametrize("rc", [False, True], ids=["k9", "remove_center"])
def test_autograd_function_bf16(rc):
    """dcn_core in bf16 through torch autograd (the 16-bit backward with a
    workspace from torch's allocator), against the oracle on the 16-bit gate."""
    wl = BWD16[2].replace(dtype="bf16", remove_center=rc)
    t = synth.make_inputs(wl, with_grad=True)
    x, off, m, gy = (t[k].to(DEV).requires_grad_(k != "grad_out") for k in ("x", "offset", "mask", "grad_out"))
    y = dcn.dcn_core(x, off, m, **wl.op_kwargs())
    gx, goff, gm = torch.autograd.grad(y, (x, off, m), grad_outputs=gy)
    assert gx.dtype == torch.bfloat16
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(y.detach()), oracle_full(wl, t), "bf16", f"autograd bf16 rc={rc} output")
    gate(_np(gx), rx, "bf16", f"autograd bf16 rc={rc} grad_input")
    gate(_np(goff), roff, "bf16", f"autograd bf16 rc={rc} grad_offset")
    gate(_np(gm), rm, "bf16", f"autograd bf16 rc={rc} grad_mask")


# --------------------------------------------------------------------------- edge cases

def test_empty_batch():
    x = torch.empty(0, 8, 8, 16, device=DEV)
    off = torch.empty(0, 8, 8, 1, 9, 2, device=DEV)
    m = torch.empty(0, 8, 8, 1, 9, device=DEV)
    y = dcn.dcn_forward(x, off, m, groups=1)
    assert y.shape == (0, 8, 8, 16)
    gx, goff, gm = dcn.dcn_backward(x, off, m, torch.empty(0, 8, 8, 16, device=DEV), groups=1)
    assert gx.shape == x.shape and goff.shape == off.shape and gm.shape == m.shape


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_far_offsets_give_exact_zeros(dtype):
    wl = Workload("far", n=1, h=7, w=9, c=32, groups=2, dtype=dtype, seed=41)
    t = synth.make_inputs(wl)
    for big in (1e4, -1e4, float("inf"), -float("inf"), 3e38):
        t["offset"] = torch.full_like(t["offset"], big)
        y = run_forward(wl, t)
        assert torch.all(y == 0), big


@pytest.mark.parametrize("path", ["auto", "generic", "tiled"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_far_offsets_backward_exact_zeros(dtype, path, monkeypatch):
    """Offsets that put every sample off the map (+-1e4, +-Inf, 3e38, on both
    axes or on one): every gradient is exactly zero, as the oracle's pinned
    far-away branch gives (zero padding: B = 0 and dB = 0 off the map)."""
    if path != "auto":
        if dtype != "f32" and path == "tiled":
            pytest.skip("the half-window tiled backward is fp32 only")
        monkeypatch.setenv("DCN_MI355X_BWD_PATH", path)
    wl = Workload("far_bwd", n=2, h=19, w=21, c=32, groups=2, dtype=dtype, seed=46)
    t = synth.make_inputs(wl, with_grad=True)
    rng = np.random.default_rng(9)
    for big in (1e4, -1e4, float("inf"), -float("inf"), 3e38):
        for axes in ((0, 1), (0,), (1,)):
            off = torch.from_numpy(rng.standard_normal(t["offset"].shape).astype(np.float32))
            for a in axes:
                off[..., a] = big
            t["offset"] = off.to(t["x"].dtype)
            print(f"backward far offsets {big} axes {axes} {dtype} path={path}", flush=True)
            gx, goff, gm = run_backward(wl, t)
            rx, roff, rm = oracle_backward(wl, t)
            assert np.all(rx == 0) and np.all(roff == 0) and np.all(rm == 0)
            assert torch.all(gx == 0), (big, axes, "grad_input")
            assert torch.all(goff == 0), (big, axes, "grad_offset")
            assert torch.all(gm == 0), (big, axes, "grad_mask")


GUARD = 256  # elements of canary on each side of every output buffer


def _guarded(shape, dtype, fill):
    """A tensor of `shape` inside a buffer with GUARD canary elements on each
    side; returns (view, buffer)."""
    numel = int(np.prod(shape))
    buf = torch.full((numel + 2 * GUARD,), fill, dtype=dtype, device=DEV)
    return buf[GUARD:GUARD + numel].view(shape), buf


def _canaries_intact(buf, fill, what):
    head, tail = buf[:GUARD], buf[-GUARD:]
    assert torch.all(head == fill) and torch.all(tail == fill), f"{what}: a guard band was written"


@pytest.mark.parametrize("small", [False, True], ids=["tiles", "whole_map"])
@pytest.mark.parametrize("path", ["auto", "generic", "tiled"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_guard_bands_untouched(dtype, path, small, monkeypatch):
    """grad_input, grad_offset, grad_mask and the 16-bit fp32 workspace each
    sit between two guard bands of canary values; a multi-tile problem whose
    offsets reach far outside the tile windows and the map (the global
    fix-up and atomic paths) must leave every band as it was, call after
    call, and give the oracle's gradients."""
    if path != "auto":
        if dtype != "f32" and path == "tiled":
            pytest.skip("the half-window tiled backward is fp32 only")
        monkeypatch.setenv("DCN_MI355X_BWD_PATH", path)
    wl = Workload("guard_bwd", n=2, h=37, w=29, c=48, groups=3, dtype=dtype, offset_dist=uniform(8.0), seed=47)
    if small:  # the whole-map kernel's shapes
        wl = wl.replace(h=21, w=19)
    t = synth.make_inputs(wl, with_grad=True)
    x, off, m, gy = (t[k].to(DEV) for k in ("x", "offset", "mask", "grad_out"))
    fill = 12345.0 if dtype == "f32" else 1234.0
    gx, bx = _guarded(x.shape, x.dtype, fill)
    goff, boff = _guarded(off.shape, x.dtype, fill)
    gm, bm = _guarded(m.shape, x.dtype, fill)
    need = dcn.backward_workspace_bytes(x, **wl.op_kwargs())
    ws = bws = None
    if need:
        ws, bws = _guarded((need // 4,), torch.float32, -777.0)
    rx, roff, rm = oracle_backward(wl, t)
    for call in range(2):
        print(f"backward guard bands {dtype} path={path} small={small} call {call}", flush=True)
        dcn.dcn_backward(x, off, m, gy, grad_input=gx, grad_offset=goff, grad_mask=gm,
                         workspace=None if ws is None else ws.view(torch.uint8), **wl.op_kwargs())
        torch.cuda.synchronize()
        _canaries_intact(bx, fill, "grad_input")
        _canaries_intact(boff, fill, "grad_offset")
        _canaries_intact(bm, fill, "grad_mask")
        if bws is not None:
            _canaries_intact(bws, -777.0, "workspace")
        gate(_np(gx), rx, dtype, f"guarded grad_input call {call}")
        gate(_np(goff), roff, dtype, f"guarded grad_offset call {call}")
        gate(_np(gm), rm, dtype, f"guarded grad_mask call {call}")


@pytest.mark.parametrize("ks", [3, 5, "map"], ids=["k3", "k5", "k3_whole_map"])
@pytest.mark.parametrize("path", ["auto", "tiled"])
@pytest.mark.parametrize("softmax", [True, False], ids=["dcnv3_gy_outlier", "dcnv4_mask_outlier"])
def test_backward_outlier_per_tile(softmax, path, ks, monkeypatch):
    """Heavy-tailed gradients: in every other 16x16 output tile one
    pixel-group carries terms 1e4 times the others (DCNv3: its grad_output
    row scaled by 1e4; DCNv4: its unnormalised mask row).  grad_input
    elements that none of those pixel-groups' samples reach keep the fp32
    bar of 1e-4 against the oracle; elements they reach are held to 1e-4 of
    their sum of absolute terms (the oracle's grad_input with |grad_output|
    and |mask|); the outliers' own offset and mask rows to 1e-4 of their
    largest value, and every other offset and mask gradient to 1e-4."""
    monkeypatch.setenv("DCN_MI355X_BWD_PATH", path)
    hw = (24, 24) if ks == "map" else (48, 40)  # 24x24: the whole-map kernel, its items on atomics
    ks = 3 if ks == "map" else ks
    wl = Workload("outlier", n=2, h=hw[0], w=hw[1], c=32, groups=2, softmax=softmax, kernel=(ks, ks),
                  pad=(ks // 2, ks // 2), mask_dist=normal(1.0 if softmax else 0.5), offset_dist=normal(1.5),
                  seed=48)
    t = synth.make_inputs(wl, with_grad=True)
    rng = np.random.default_rng(10)
    ho, wo = wl.out_hw
    hot = []  # (n, ho, wo, g) of the outliers
    for n in range(wl.n):
        for g in range(wl.groups):
            for ty in range(0, ho, 16):
                for tx in range(0, wo, 16):
                    if (ty // 16 + tx // 16 + g) % 2 == 0:
                        hot.append((n, int(rng.integers(ty, min(ty + 16, ho))),
                                    int(rng.integers(tx, min(tx + 16, wo))), g))
    for (n, y, xx, g) in hot:
        if softmax:
            t["grad_out"][n, y, xx, 16 * g:16 * g + 16] *= 1e4
        else:
            t["mask"][n, y, xx, g] *= 1e4
    print(f"backward outliers softmax={softmax} path={path} {ks}x{ks} ({len(hot)} outliers)", flush=True)
    gx, goff, gm = (_np(a) for a in run_backward(wl, t))
    rx, roff, rm = oracle_backward(wl, t)
    # the outliers' scatter alone (grad_output zero elsewhere) marks the
    # grad_input elements they reach
    keep = torch.zeros(t["grad_out"].shape, dtype=torch.bool)
    for (n, y, xx, g) in hot:
        keep[n, y, xx, 16 * g:16 * g + 16] = True
    only = dict(t, grad_out=torch.where(keep, t["grad_out"], torch.zeros_like(t["grad_out"])))
    reach = np.abs(oracle_backward(wl, only)[0]) > 0
    assert reach.any() and not reach.all()
    # sum of the absolute scatter terms of every element
    absd = dict(t, grad_out=t["grad_out"].abs(), mask=t["mask"] if softmax else t["mask"].abs())
    scale = oracle_backward(wl, absd)[0]
    err = np.abs(gx - rx)
    assert err[~reach].max() <= ATOL_F32, f"grad_input away from the outliers: {err[~reach].max():.3e}"
    worst = float(np.max(err[reach] / np.maximum(1.0, scale[reach])))
    assert worst <= 1e-4, f"grad_input near the outliers: {worst:.3e} of the absolute terms"
    rows = np.zeros(rm.shape[:4], dtype=bool)
    for h_ in hot:
        rows[h_] = True
    for got, ref, name in ((goff, roff, "grad_offset"), (gm, rm, "grad_mask")):
        e = np.abs(got - ref).reshape(rows.shape + (-1,))
        r = np.abs(ref).reshape(rows.shape + (-1,))
        assert e[~rows].max() <= ATOL_F32, f"{name} of ordinary pixel-groups: {e[~rows].max():.3e}"
        rowmax = np.maximum(1.0, r[rows].max(axis=-1, keepdims=True))
        assert np.all(e[rows] <= 1e-4 * rowmax), f"{name} of the outliers"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_backward_whole_map_atomic_items_16bit(dtype):
    """16-bit I/O on the whole-map backward with a few grad_output rows
    scaled by 1000: those items' terms are too spread for fixed point, so
    they clear their slice of the caller's fp32 workspace, add there with
    fp32 atomics and round the slice into grad_input; every gradient within
    the 16-bit bar of the oracle."""
    wl = Workload("map_atomics", n=2, h=20, w=17, c=48, groups=3, dtype=dtype, offset_dist=normal(2.0), seed=63)
    t = synth.make_inputs(wl, with_grad=True)
    ho, wo = wl.out_hw
    for (n, y, x, g) in ((0, 3, 4, 0), (0, 15, 11, 1), (1, 8, 2, 2), (1, 19, 16, 0)):
        t["grad_out"][n, y, x, 16 * g:16 * g + 16] *= 1000
    print(f"backward whole-map atomic items {dtype}", flush=True)
    gx, goff, gm = run_backward(wl, t)
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(gx), rx, dtype, f"map atomics {dtype} grad_input")
    gate(_np(goff), roff, dtype, f"map atomics {dtype} grad_offset")
    gate(_np(gm), rm, dtype, f"map atomics {dtype} grad_mask")


def test_nan_offset_poisons_only_its_group():
    wl = Workload("nan", n=1, h=6, w=5, c=32, groups=2, seed=42)
    t = synth.make_inputs(wl, with_grad=True)
    t["offset"][0, 2, 3, 1, 4, 0] = float("nan")
    y = _np(run_forward(wl, t))
    gate(y, oracle_full(wl, t), "f32", "nan offset forward")
    assert np.isnan(y[0, 2, 3, 16:]).all() and np.isfinite(y).sum() == y.size - 16
    gx, goff, gm = run_backward(wl, t)
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(gx), rx, "f32", "nan offset grad_input")
    gate(_np(goff), roff, "f32", "nan offset grad_offset")
    gate(_np(gm), rm, "f32", "nan offset grad_mask")


def test_nan_input_propagates():
    wl = Workload("nan_in", n=1, h=6, w=6, c=16, groups=1, seed=43)
    t = synth.make_inputs(wl)
    # integer s*offset = 0 everywhere: every sample hits pixel centres with
    # weight exactly 1 at one corner, so the NaN reaches exactly the outputs
    # whose 3x3 window covers it
    t["offset"].zero_()
    t["x"][0, 2, 3, 5] = float("nan")
    y = _np(run_forward(wl, t))
    ref = oracle_full(wl, t)
    # corners with weight exactly 0 may or may not read the NaN: compare only
    # where the oracle is finite, and require NaN where the oracle is NaN
    assert np.all(np.isnan(y[np.isnan(ref)]))
    fin = np.isfinite(ref) & np.isfinite(y)
    assert np.abs(y[fin] - ref[fin]).max() <= ATOL_F32


def test_integer_offsets_are_exact_gathers():
    wl = Workload("int", n=2, h=11, w=9, c=32, groups=2, softmax=False, seed=44)
    t = synth.make_inputs(wl)
    rng = np.random.default_rng(5)
    t["offset"] = torch.from_numpy((rng.integers(-3, 4, size=t["offset"].shape) / 2.0).astype(np.float32))
    t["mask"] = torch.ones_like(t["mask"])
    y = _np(run_forward(wl, t))
    # with unit weights and pixel-centre samples the only rounding is the
    # fp32 sum of 9 input values
    assert np.abs(y - oracle_full(wl, t)).max() <= 4e-6


def test_output_guard_bands_untouched():
    wl = Workload("guard", n=2, h=9, w=7, c=48, groups=3, seed=45)
    t = synth.make_inputs(wl)
    x, off, m = (t[k].to(DEV) for k in ("x", "offset", "mask"))
    numel = wl.n * wl.out_hw[0] * wl.out_hw[1] * wl.c
    pad = 1024
    buf = torch.full((numel + 2 * pad,), 12345.0, device=DEV)
    out = buf[pad:pad + numel].view(wl.n, *wl.out_hw, wl.c)
    dcn.dcn_forward(x, off, m, out=out, **wl.op_kwargs())
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[pad + numel:] == 12345.0)
    gate(_np(out), oracle_full(wl, t), "f32", "guarded output")


def test_forward_is_deterministic():
    wl = synth.WORKLOADS["hires_dcnv3_f32"]
    t = synth.make_inputs(wl, with_grad=False)
    a = run_forward(wl, t)
    b = run_forward(wl, t)
    assert torch.equal(a, b)


def test_runs_on_a_side_stream():
    wl = SMALL[0]
    t = synth.make_inputs(wl)
    x, off, m = (t[k].to(DEV) for k in ("x", "offset", "mask"))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = dcn.dcn_forward(x, off, m, **wl.op_kwargs())
    s.synchronize()
    gate(_np(y), oracle_full(wl, t), "f32", "side stream")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_graph_capture_replays_match_eager(dtype):
    """Forward and backward captured in a HIP graph (the library clears with a
    fill kernel, never hipMemsetAsync): every replay, on new inputs copied into
    the captured buffers with eager work and a synchronisation between
    replays, equals an eager call on the same inputs."""
    wl = PATH_CASES[0].replace(dtype=dtype)
    kw = wl.op_kwargs()
    print(f"graph capture {dtype}", flush=True)
    draws = [synth.make_inputs(wl.replace(seed=wl.seed + 100 * r), with_grad=True) for r in range(4)]
    x, off, m, gy = (draws[0][k].to(DEV) for k in ("x", "offset", "mask", "grad_out"))
    y = torch.empty((wl.n, *wl.out_hw, wl.c), dtype=x.dtype, device=DEV)
    gx, goff, gm = torch.empty_like(x), torch.empty_like(off), torch.empty_like(m)
    nb = dcn.backward_workspace_bytes(x, **kw)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    outs = dict(grad_input=gx, grad_offset=goff, grad_mask=gm, workspace=ws if nb else None)

    def step():
        dcn.dcn_forward(x, off, m, out=y, **kw)
        dcn.dcn_backward(x, off, m, gy, **outs, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(1, 4):
        for k, dst in (("x", x), ("offset", off), ("mask", m), ("grad_out", gy)):
            dst.copy_(draws[r][k].to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [_np(t) for t in (y, gx, goff, gm)]
        ey = dcn.dcn_forward(x, off, m, **kw)
        eg = dcn.dcn_backward(x, off, m, gy, **kw)
        torch.cuda.synchronize()
        ref = [_np(ey)] + [_np(t) for t in eg]
        # the forward is deterministic; grad_input's fp32 atomics may add in another order
        assert np.array_equal(got[0], ref[0]), f"replay {r}: output"
        assert np.array_equal(got[2], ref[2]) and np.array_equal(got[3], ref[3]), f"replay {r}: grad_offset/mask"
        tol = 1e-5 if dtype == "f32" else 2.0 ** -7
        np.testing.assert_allclose(got[1], ref[1], rtol=tol, atol=1e-5, err_msg=f"replay {r}: grad_input")


def test_concurrent_calls_from_two_threads():
    """The library keeps no mutable state: two host threads, each on its own
    stream, run forwards of different problems at once and get the results
    of serial calls."""
    import threading
    cases = [PATH_CASES[0], PATH_CASES[3].replace(dtype="bf16")]
    ins = [{k: v.to(DEV) for k, v in synth.make_inputs(wl).items()} for wl in cases]
    ref = [_np(dcn.dcn_forward(t["x"], t["offset"], t["mask"], **wl.op_kwargs())) for wl, t in zip(cases, ins)]
    torch.cuda.synchronize()
    got = [None, None]
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(20):
                    y = dcn.dcn_forward(ins[i]["x"], ins[i]["offset"], ins[i]["mask"], **cases[i].op_kwargs())
            s.synchronize()
            got[i] = _np(y)
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not errors, errors
    for i in range(2):
        assert np.array_equal(got[i], ref[i]), f"thread {i}"


# Each group's mask is dominated by one point: DCNv3 logits 0 at that point
# and -30 elsewhere (a softmax weight of 1 - 8e-13), DCNv4 a one-hot mask.
# The pairs cover the points that the group-pair kernels assign specially
# (the first group's point 8 and the second group's point 0 ride in one
# 16-byte chunk; lane 0 takes logit 8 from lane 3), so a point read from the
# wrong group, slot or lane shows as a wrong sample, not a small drift.
DOMINANT = [(8, 0), (0, 8), (8, 8), (0, 0), (4, 4), (7, 1), (1, 7)]


def _dominated_mask(wl, t, points, softmax):
    m = torch.full_like(t["mask"], -30.0 if softmax else 0.0)
    for g in range(wl.groups):
        m[..., g, points[g % 2]] = 0.0 if softmax else 1.0
    return m


@pytest.mark.parametrize("softmax", [True, False], ids=["dcnv3", "dcnv4"])
@pytest.mark.parametrize("groups", [2, 4])
@pytest.mark.parametrize("points", DOMINANT, ids=lambda p: f"p{p[0]}_{p[1]}")
def test_pair_kernels_point_ownership(points, groups, softmax, monkeypatch):
    wl = Workload("own", n=1, h=21, w=19, c=16 * groups, groups=groups, softmax=softmax,
                  offset_dist=normal(2.0), seed=60 + groups)
    print(f"ownership {points} groups={groups} softmax={softmax}", flush=True)
    t = synth.make_inputs(wl, with_grad=True)
    t["mask"] = _dominated_mask(wl, t, points, softmax)
    monkeypatch.setenv("DCN_MI355X_FWD_PATH", "pair")
    gate(_np(run_forward(wl, t)), oracle_full(wl, t), "f32", f"own {points} forward")
    monkeypatch.setenv("DCN_MI355X_BWD_PATH", "quad")
    gx, goff, gm = run_backward(wl, t)
    rx, roff, rm = oracle_backward(wl, t)
    gate(_np(gx), rx, "f32", f"own {points} grad_input")
    gate(_np(goff), roff, "f32", f"own {points} grad_offset")
    gate(_np(gm), rm, "f32", f"own {points} grad_mask")
