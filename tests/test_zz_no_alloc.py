"""dcn_backward_noalloc, the backward entry point that allocates nothing, on
the GPU through the C ABI: its results against dcn_backward's (the entry
point with a caller workspace) on the same inputs, on two calls in a row,
the second with a smaller problem, so that what the first call left in the
library's fixed scratch must not leak into the second.

The bar is the parity bar: grad_offset and grad_mask come out of the same
kernels in the same order and must be bit for bit equal; grad_input is
summed with fp32 atomics in either call, so only its rounding may differ
(one ulp of the I/O dtype after the final rounding, or fp32 rounding of the
partial sums), and both calls are also held to the oracle's gate.
"""
import numpy as np
import pytest
import torch

import deformable_convolution_vision_dcn_amd as dcn
from deformable_convolution_vision_dcn_amd import _capi, synth
from deformable_convolution_vision_dcn_amd.synth import Workload, normal, uniform
from test_parity_gpu import DEV, _np, gate, oracle_backward

pytestmark = pytest.mark.gpu


def _call_noalloc(wl, ins, outs):
    """dcn_backward_noalloc straight through the C ABI (ctypes) on torch's
    current stream, into preallocated gradient tensors."""
    p = dcn.make_problem(ins["x"].shape, dtype=ins["x"].dtype, **wl.op_kwargs())
    st = _capi.dcn_backward_noalloc(p, ins["x"].data_ptr(), ins["offset"].data_ptr(), ins["mask"].data_ptr(),
                                    ins["grad_out"].data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(),
                                    outs[2].data_ptr(), torch.cuda.current_stream(DEV).cuda_stream)
    _capi.raise_on(st)


def _check_pair(wl, ins, got, ref):
    ga, gb = (_np(g) for g in got), (_np(g) for g in ref)
    ga, gb = list(ga), list(gb)
    assert np.array_equal(ga[1], gb[1], equal_nan=True), f"{wl.name}: grad_offset differs"
    assert np.array_equal(ga[2], gb[2], equal_nan=True), f"{wl.name}: grad_mask differs"
    if wl.dtype == "f32":
        np.testing.assert_allclose(ga[0], gb[0], rtol=1e-5, atol=1e-5, err_msg=f"{wl.name}: grad_input")
    else:
        np.testing.assert_allclose(ga[0], gb[0], rtol=2.0 ** -7, atol=1e-5, err_msg=f"{wl.name}: grad_input")


# The first problem needs several chunks of images through the 64 MiB scratch
# (a 96x96x160 bf16 image has a 5.9 MB fp32 accumulator: 11 images a chunk);
# the second is smaller and of another shape (stride 2, a 3x5 kernel) and
# runs on the untiled kernel.
CASES = [
    (Workload("na_stage1_bf16", n=32, h=96, w=96, c=160, groups=10, dtype="bf16",
              offset_dist=normal(1.5), seed=81),
     Workload("na_small_f16_s2", n=3, h=21, w=19, c=48, groups=3, dtype="f16", kernel=(3, 5),
              pad=(1, 2), stride=(2, 1), softmax=False, mask_dist=normal(0.5),
              offset_dist=uniform(3.0), seed=82)),
    (Workload("na_hires_f32", n=2, h=160, w=160, c=160, groups=10, offset_dist=normal(2.0), seed=83),
     Workload("na_small_f32", n=1, h=37, w=29, c=48, groups=3, offset_dist=uniform(4.0), seed=84)),
]


@pytest.mark.parametrize("first,second", CASES, ids=lambda w: w.name)
def test_noalloc_matches_backward_on_two_calls(first, second):
    for wl in (first, second):
        print(f"noalloc backward {wl.name} {wl.dtype} n={wl.n}", flush=True)
        t = synth.make_inputs(wl, with_grad=True)
        ins = {k: v.to(DEV) for k, v in t.items()}
        outs = (torch.full_like(ins["x"], 7.0), torch.full_like(ins["offset"], 7.0),
                torch.full_like(ins["mask"], 7.0))
        _call_noalloc(wl, ins, outs)
        ref = dcn.dcn_backward(ins["x"], ins["offset"], ins["mask"], ins["grad_out"], **wl.op_kwargs())
        torch.cuda.synchronize()
        _check_pair(wl, ins, outs, ref)
        if wl.n * wl.h * wl.w <= 4096:  # small enough for the whole oracle backward
            rx, roff, rm = oracle_backward(wl, t)
            for g, r, name in zip(outs, (rx, roff, rm), ("grad_input", "grad_offset", "grad_mask")):
                gate(_np(g), r, wl.dtype, f"{wl.name} noalloc {name}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_noalloc_whole_map_items_on_atomics(dtype):
    """Small maps run the whole-map backward, whose items off fixed point add
    their terms into the fixed scratch (each first clearing its own slice):
    a few grad_output rows scaled by 2000 send items there, on two calls in a
    row, the second smaller and of another shape; each call against
    dcn_backward and the oracle."""
    wls = (Workload("na_map_24", n=4, h=24, w=24, c=64, groups=4, dtype=dtype, offset_dist=uniform(3.0), seed=85),
           Workload("na_map_12", n=2, h=12, w=11, c=32, groups=2, dtype=dtype, softmax=False,
                    mask_dist=normal(0.5), offset_dist=normal(2.0), seed=86))
    for wl in wls:
        print(f"noalloc whole-map backward {wl.name} {dtype}", flush=True)
        t = synth.make_inputs(wl, with_grad=True)
        for n in range(wl.n):
            t["grad_out"][n, 3 + n, 4, :16] *= 2000  # group 0 of image n off fixed point
        ins = {k: v.to(DEV) for k, v in t.items()}
        outs = (torch.full_like(ins["x"], 7.0), torch.full_like(ins["offset"], 7.0),
                torch.full_like(ins["mask"], 7.0))
        _call_noalloc(wl, ins, outs)
        ref = dcn.dcn_backward(ins["x"], ins["offset"], ins["mask"], ins["grad_out"], **wl.op_kwargs())
        torch.cuda.synchronize()
        _check_pair(wl, ins, outs, ref)
        rx, roff, rm = oracle_backward(wl, t)
        for g, r, name in zip(outs, (rx, roff, rm), ("grad_input", "grad_offset", "grad_mask")):
            gate(_np(g), r, wl.dtype, f"{wl.name} noalloc {name}")


def test_noalloc_whole_map_in_chunks():
    """A stage-3-shaped bf16 batch of 100 images (24x24, C = 640) runs the
    whole-map backward in three chunks through the fixed scratch (45 images
    of fp32 accumulator a chunk), dcn_backward in one: the gradients are
    equal bit for bit (integer sums, plain stores), and two images of each
    chunk match the oracle."""
    wl = Workload("na_map_chunks", n=100, h=24, w=24, c=640, groups=40, dtype="bf16", offset_dist=uniform(3.0),
                  seed=87)
    t = synth.make_inputs(wl, with_grad=True)
    ins = {k: v.to(DEV) for k, v in t.items()}
    per_chunk = _capi.NOALLOC_SCRATCH_BYTES // (wl.h * wl.w * wl.c * 4)
    assert per_chunk < wl.n < 3 * per_chunk, per_chunk
    print(f"noalloc whole-map backward in chunks of {per_chunk} images", flush=True)
    outs = (torch.full_like(ins["x"], 7.0), torch.full_like(ins["offset"], 7.0),
            torch.full_like(ins["mask"], 7.0))
    _call_noalloc(wl, ins, outs)
    ref = dcn.dcn_backward(ins["x"], ins["offset"], ins["mask"], ins["grad_out"], **wl.op_kwargs())
    torch.cuda.synchronize()
    for g, r, name in zip(outs, ref, ("grad_input", "grad_offset", "grad_mask")):
        assert torch.equal(g, r), f"{name} differs between the chunked and the single call"
    for n in (0, per_chunk - 1, per_chunk, 2 * per_chunk, wl.n - 1):
        one = wl.replace(n=1)
        tn = {k: v[n:n + 1] for k, v in t.items()}
        rx, roff, rm = oracle_backward(one, tn)
        for g, r, name in zip(outs, (rx, roff, rm), ("grad_input", "grad_offset", "grad_mask")):
            gate(_np(g[n:n + 1]), r, wl.dtype, f"image {n} {name}")


def test_noalloc_python_entry_point_and_scratch_limit():
    """The binding's dcn_backward_noalloc gives the same gradients, and a
    16-bit image whose fp32 accumulator exceeds the scratch is refused with
    DCN_ERR_SCRATCH (checked on the host: nothing is enqueued)."""
    wl = CASES[0][1]
    t = synth.make_inputs(wl, with_grad=True)
    ins = {k: v.to(DEV) for k, v in t.items()}
    got = dcn.dcn_backward_noalloc(ins["x"], ins["offset"], ins["mask"], ins["grad_out"], **wl.op_kwargs())
    ref = dcn.dcn_backward(ins["x"], ins["offset"], ins["mask"], ins["grad_out"], **wl.op_kwargs())
    torch.cuda.synchronize()
    _check_pair(wl, ins, got, ref)
    big = torch.empty(1, 2048, 2048, 16, dtype=torch.bfloat16, device=DEV)
    assert big[0].numel() * 4 > _capi.NOALLOC_SCRATCH_BYTES
    off = torch.empty(1, 2048, 2048, 1, 9, 2, dtype=torch.bfloat16, device=DEV)
    m = torch.empty(1, 2048, 2048, 1, 9, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dcn.DCNError, match="DCN_ERR_SCRATCH"):
        dcn.dcn_backward_noalloc(big, off, m, big, groups=1, grad_input=torch.empty_like(big),
                                 grad_offset=torch.empty_like(off), grad_mask=torch.empty_like(m))
