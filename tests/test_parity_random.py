"""Seeded random problems against the oracle.

Each seed draws one problem -- batch, map size (1 to 40 on a side), groups,
kernel size, stride, dilation, pad, offset scale, offset spread (from nearly
integer-free small offsets to ones that leave any window), DCNv3 or DCNv4,
dtype -- and runs the forward on every kernel in turn (forced through
DCN_MI355X_FWD_PATH; a kernel that does not apply falls back to the generic
one) and, for fp32, the backward on every backward kernel.  The bar is the
same as the fixed cases: max-abs 1e-4 in fp32, |d| <= 2e-2 |ref| + 1e-3 for
16-bit outputs.  The 16-bit draws also run the 16-bit backward on every
backward kernel that takes them (default and untiled), and a second series
of draws, held to the tiled backward's shape (3x3 points at stride 1), runs
it on the tiled kernel.
"""
import numpy as np
import pytest

from deformable_convolution_vision_dcn_amd import synth
from deformable_convolution_vision_dcn_amd.synth import Workload, normal, uniform
from test_parity_gpu import _np, gate, oracle_backward, oracle_full, run_backward, run_forward

pytestmark = pytest.mark.gpu

SEEDS = range(36)
FWD_PATHS = ["auto", "generic", "tiled", "pair", "lane", "map"]
BWD_PATHS = ["auto", "generic", "tiled", "quad"]


def random_problem(seed: int) -> Workload:
    r = np.random.default_rng(7000 + seed)
    dtype = ("f32", "f16", "bf16")[seed % 3]
    kernel = [(3, 3)] * 6 + [(1, 1), (3, 5), (5, 5)]
    kh, kw = kernel[int(r.integers(0, len(kernel)))]
    stride = (int(r.choice([1, 1, 1, 2])), int(r.choice([1, 1, 1, 2])))
    dil = (int(r.choice([1, 1, 2])), int(r.choice([1, 1, 2])))
    pad = (int(r.integers(0, 3)), int(r.integers(0, 3)))
    h, w = int(r.integers(1, 41)), int(r.integers(1, 41))
    # grow the map until the output has at least one pixel
    h = max(h, dil[0] * (kh - 1) + 1 - 2 * pad[0])
    w = max(w, dil[1] * (kw - 1) + 1 - 2 * pad[1])
    groups = int(r.integers(1, 5))
    spread = float(r.choice([0.3, 1.5, 4.0, 10.0]))
    offset_dist = normal(spread) if r.integers(0, 2) else uniform(spread)
    softmax = bool(r.integers(0, 2))
    # every fourth draw with an odd kernel of several points drops the centre
    rc = seed % 4 == 3 and kh % 2 == 1 and kw % 2 == 1 and kh * kw > 1
    return Workload(f"rand{seed}", n=int(r.integers(1, 4)), h=h, w=w, c=16 * groups, groups=groups,
                    remove_center=rc,
                    dtype=dtype, softmax=softmax, kernel=(kh, kw), stride=stride, pad=pad,
                    dilation=dil, offset_scale=float(r.choice([0.5, 1.0, 2.0])),
                    offset_dist=offset_dist, mask_dist=normal(1.0 if softmax else 0.5), seed=seed)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_forward_every_kernel(seed, monkeypatch):
    wl = random_problem(seed)
    t = synth.make_inputs(wl)
    ref = oracle_full(wl, t)
    for path in FWD_PATHS:
        if path == "auto":
            monkeypatch.delenv("DCN_MI355X_FWD_PATH", raising=False)
        else:
            monkeypatch.setenv("DCN_MI355X_FWD_PATH", path)
        print(f"forward {wl} path={path}", flush=True)
        gate(_np(run_forward(wl, t)), ref, wl.dtype, f"{wl.name}/{wl.dtype}/{path}")


@pytest.mark.parametrize("seed", [s for s in SEEDS if s % 3 == 0])  # the fp32 draws
def test_random_backward_every_kernel(seed, monkeypatch):
    wl = random_problem(seed)
    assert wl.dtype == "f32"
    t = synth.make_inputs(wl, with_grad=True)
    rx, roff, rm = oracle_backward(wl, t)
    for path in BWD_PATHS:
        if path == "auto":
            monkeypatch.delenv("DCN_MI355X_BWD_PATH", raising=False)
        else:
            monkeypatch.setenv("DCN_MI355X_BWD_PATH", path)
        print(f"backward {wl} path={path}", flush=True)
        gx, goff, gm = run_backward(wl, t)
        gate(_np(gx), rx, "f32", f"{wl.name}/{path} grad_input")
        gate(_np(goff), roff, "f32", f"{wl.name}/{path} grad_offset")
        gate(_np(gm), rm, "f32", f"{wl.name}/{path} grad_mask")



@pytest.mark.parametrize("seed", [s for s in SEEDS if s % 3 != 0])  # the 16-bit draws
def test_random_backward_16bit_any_shape(seed, monkeypatch):
    wl = random_problem(seed)
    assert wl.dtype in ("f16", "bf16")
    t = synth.make_inputs(wl, with_grad=True)
    rx, roff, rm = oracle_backward(wl, t)
    for path in ["auto", "generic"]:
        if path == "auto":
            monkeypatch.delenv("DCN_MI355X_BWD_PATH", raising=False)
        else:
            monkeypatch.setenv("DCN_MI355X_BWD_PATH", path)
        print(f"backward {wl} path={path}", flush=True)
        gx, goff, gm = run_backward(wl, t)
        gate(_np(gx), rx, wl.dtype, f"{wl.name}/{wl.dtype}/{path} grad_input")
        gate(_np(goff), roff, wl.dtype, f"{wl.name}/{wl.dtype}/{path} grad_offset")
        gate(_np(gm), rm, wl.dtype, f"{wl.name}/{wl.dtype}/{path} grad_mask")


def random_problem_16(seed: int) -> Workload:
    """A draw of random_problem with the shape the 16-bit backward covers:
    3x3 points at stride 1 (every third without the centre, every fourth at
    dilation 2), f16 or bf16."""
    wl = random_problem(100 + seed)
    dil = 2 if seed % 4 == 1 else 1
    return wl.replace(name=f"rand16_{seed}", dtype=("f16", "bf16")[seed % 2], kernel=(3, 3),
                      remove_center=seed % 3 == 2, dilation=(dil, dil),
                      stride=(1, 1), h=max(wl.h, 2 * dil + 1 - 2 * wl.pad[0]),
                      w=max(wl.w, 2 * dil + 1 - 2 * wl.pad[1]))


@pytest.mark.parametrize("seed", range(16))
def test_random_backward_16bit(seed):
    """16-bit backward on random 3x3, stride-1 problems, on the 16-bit gate."""
    wl = random_problem_16(seed)
    t = synth.make_inputs(wl, with_grad=True)
    rx, roff, rm = oracle_backward(wl, t)
    print(f"backward {wl}", flush=True)
    gx, goff, gm = run_backward(wl, t)
    gate(_np(gx), rx, wl.dtype, f"{wl.name}/{wl.dtype} grad_input")
    gate(_np(goff), roff, wl.dtype, f"{wl.name}/{wl.dtype} grad_offset")
    gate(_np(gm), rm, wl.dtype, f"{wl.name}/{wl.dtype} grad_mask")
