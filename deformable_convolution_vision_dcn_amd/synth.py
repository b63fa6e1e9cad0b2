"""Seeded synthetic inputs for the DCN core.

This module only draws random numbers and names the workloads; it holds none
of the operator's arithmetic.  The HIP path and the CPU oracle both take their
inputs from here, and from nowhere else.

The workloads stand in for InternImage-L activations at 384x384 input
(wmrh.cn/news/61976, section 一 for the 384 input and section 四 for the stage
layout: a stem that downsamples by 4, stages of 160/320/640/1280 channels, so
stage maps of 96/48/24/12 pixels).  The groups of that model are [10, 20, 40,
80] (section 二, step 4), i.e. 16 channels per group at every stage.  No trained
offsets or masks are available, so the offsets and mask values are drawn from
the stated distributions; the second parameter of N(mu, sigma) is the standard
deviation.

Generator: numpy's PCG64 seeded with ``[seed, draw, tensor_id]``, one
independent stream per tensor (x=0, offset=1, mask=2, grad_out=3).  Values are
drawn in float32 and rounded to the I/O dtype by torch (round to nearest even).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Dist:
    """A value distribution: ('normal', std) or ('uniform', half_width)."""
    kind: str
    scale: float

    def draw(self, rng: np.random.Generator, shape) -> np.ndarray:
        if self.kind == "normal":
            a = rng.standard_normal(size=shape, dtype=np.float32)
            if self.scale != 1.0:
                a *= np.float32(self.scale)
            return a
        if self.kind == "uniform":
            a = rng.random(size=shape, dtype=np.float32)
            a *= np.float32(2.0 * self.scale)
            a -= np.float32(self.scale)
            return a
        if self.kind == "zero":
            return np.zeros(shape, dtype=np.float32)
        raise ValueError(self.kind)


def normal(std: float) -> Dist:
    return Dist("normal", float(std))


def uniform(half_width: float) -> Dist:
    return Dist("uniform", float(half_width))


ZERO = Dist("zero", 0.0)

# The output extent of a problem is part of the operator's arithmetic, which
# this module does not hold: the process drawing inputs installs a function
# workload -> (Ho, Wo) for it (the test suite and the smoke check use the
# oracle's, the benchmark the library's own host-side check).
_out_hw_fn = None


def set_out_hw(fn) -> None:
    global _out_hw_fn
    _out_hw_fn = fn


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int
    h: int
    w: int
    c: int
    groups: int
    dtype: str = "f32"
    softmax: bool = True
    kernel: Tuple[int, int] = (3, 3)
    stride: Tuple[int, int] = (1, 1)
    pad: Tuple[int, int] = (1, 1)
    dilation: Tuple[int, int] = (1, 1)
    offset_scale: float = 2.0
    x_dist: Dist = normal(1.0)
    offset_dist: Dist = normal(1.0)
    mask_dist: Dist = normal(1.0)
    grad_dist: Dist = normal(1.0)
    seed: int = 0
    draw: int = 0
    backward: bool = False
    remove_center: bool = False

    @property
    def out_hw(self) -> Tuple[int, int]:
        """Output extent (Ho, Wo), from the function installed by set_out_hw."""
        if _out_hw_fn is None:
            raise RuntimeError("synth.set_out_hw() must install the output-extent function first")
        ho, wo = _out_hw_fn(self)
        return int(ho), int(wo)

    @property
    def points(self) -> int:
        return self.kernel[0] * self.kernel[1] - (1 if self.remove_center else 0)

    @property
    def samples(self) -> int:
        """Bilinear samples per call: N*Ho*Wo*G*K."""
        ho, wo = self.out_hw
        return self.n * ho * wo * self.groups * self.points

    def shapes(self) -> Dict[str, tuple]:
        ho, wo = self.out_hw
        K = self.points
        return {
            "x": (self.n, self.h, self.w, self.c),
            "offset": (self.n, ho, wo, self.groups, K, 2),
            "mask": (self.n, ho, wo, self.groups, K),
            "grad_out": (self.n, ho, wo, self.c),
        }

    def op_kwargs(self) -> dict:
        """Keyword arguments describing the operator (shared spelling of both sides)."""
        kw = dict(groups=self.groups, kernel=self.kernel, stride=self.stride, pad=self.pad,
                  dilation=self.dilation, offset_scale=self.offset_scale, softmax=self.softmax)
        if self.remove_center:
            kw["remove_center"] = True
        return kw

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The named workloads: one small case and four InternImage-L-shaped ones.
WORKLOADS: Dict[str, Workload] = {
    "tiny_dcnv3_f32": Workload(
        "tiny_dcnv3_f32", n=1, h=8, w=8, c=16, groups=1, dtype="f32", softmax=True,
        offset_dist=uniform(2.0), seed=0),
    "stage1_dcnv3_f32": Workload(
        "stage1_dcnv3_f32", n=32, h=96, w=96, c=160, groups=10, dtype="f32", softmax=True,
        offset_dist=normal(1.5), seed=1),
    "stage3_dcnv3_bf16": Workload(
        "stage3_dcnv3_bf16", n=128, h=24, w=24, c=640, groups=40, dtype="bf16", softmax=True,
        offset_dist=uniform(3.0), seed=2),
    "stage2_dcnv4_f16": Workload(
        "stage2_dcnv4_f16", n=64, h=48, w=48, c=320, groups=20, dtype="f16", softmax=False,
        offset_dist=normal(1.0), mask_dist=normal(0.5), seed=3, draw=0),
    "stage4_dcnv4_f16": Workload(
        "stage4_dcnv4_f16", n=64, h=12, w=12, c=1280, groups=80, dtype="f16", softmax=False,
        offset_dist=normal(1.0), mask_dist=normal(0.5), seed=3, draw=1),
    "hires_dcnv3_f32": Workload(
        "hires_dcnv3_f32", n=2, h=160, w=160, c=160, groups=10, dtype="f32", softmax=True,
        offset_dist=normal(2.0), seed=4, backward=True),
}

HEADLINE = "stage1_dcnv3_f32"

_TENSOR_IDS = {"x": 0, "offset": 1, "mask": 2, "grad_out": 3}


def draw_tensor(wl: Workload, name: str, dist: Optional[Dist] = None) -> torch.Tensor:
    """One input tensor of ``wl`` on the CPU, in the workload's I/O dtype."""
    shape = wl.shapes()[name]
    if dist is None:
        dist = {"x": wl.x_dist, "offset": wl.offset_dist, "mask": wl.mask_dist,
                "grad_out": wl.grad_dist}[name]
    rng = np.random.default_rng([wl.seed, wl.draw, _TENSOR_IDS[name]])
    a = dist.draw(rng, shape)
    t = torch.from_numpy(a)
    return t if wl.dtype == "f32" else t.to(DTYPES[wl.dtype])


def make_inputs(wl: Workload, with_grad: Optional[bool] = None) -> Dict[str, torch.Tensor]:
    """All inputs of ``wl`` (CPU tensors, I/O dtype): x, offset, mask [, grad_out]."""
    if with_grad is None:
        with_grad = wl.backward
    names = ["x", "offset", "mask"] + (["grad_out"] if with_grad else [])
    return {k: draw_tensor(wl, k) for k in names}


# --------------------------------------------------------------------------- the fused forwards
_EXTRA_IDS = {"guide": 4, "w_offset": 5, "b_offset": 6, "w_mask": 7, "b_mask": 8, "w_out": 9, "b_out": 10}


def _std(d: Dist) -> float:
    return d.scale if d.kind == "normal" else d.scale / 3 ** 0.5


def _extra(wl: Workload, name: str, shape, std: float) -> torch.Tensor:
    rng = np.random.default_rng([wl.seed, wl.draw, _EXTRA_IDS[name]])
    a = normal(std).draw(rng, shape)
    t = torch.from_numpy(a)
    return t if wl.dtype == "f32" else t.to(DTYPES[wl.dtype])


def make_generation_inputs(wl: Workload, guide_channels: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """The guide feature (N, Ho, Wo, Cgd) ~ N(0, 1) and the two linear
    branches that turn it into offsets and mask values (CPU tensors, I/O
    dtype).  The weights are N(0, sd / sqrt(Cgd)) and the biases
    N(0, sd / 10), sd the spread of the workload's own offset and mask draws,
    so the generated values have about that spread."""
    cgd = guide_channels or wl.c
    ho, wo = wl.out_hw
    K = wl.points
    so, sm = _std(wl.offset_dist), _std(wl.mask_dist)
    return {
        "guide": _extra(wl, "guide", (wl.n, ho, wo, cgd), 1.0),
        "w_offset": _extra(wl, "w_offset", (wl.groups * K * 2, cgd), so / cgd ** 0.5),
        "b_offset": _extra(wl, "b_offset", (wl.groups * K * 2,), so / 10),
        "w_mask": _extra(wl, "w_mask", (wl.groups * K, cgd), sm / cgd ** 0.5),
        "b_mask": _extra(wl, "b_mask", (wl.groups * K,), sm / 10),
    }


def make_projection_inputs(wl: Workload) -> Dict[str, torch.Tensor]:
    """The output_proj weights (C, C) ~ N(0, 1 / sqrt(C)) and bias
    ~ N(0, 0.1) (CPU tensors, I/O dtype)."""
    return {"w_out": _extra(wl, "w_out", (wl.c, wl.c), 1.0 / wl.c ** 0.5),
            "b_out": _extra(wl, "b_out", (wl.c,), 0.1)}
