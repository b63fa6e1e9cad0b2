"""torch-tensor entry points with the C ABI's names.

Marshalling only: shapes, dtypes, devices and contiguity are checked here (the
C ABI receives bare pointers and cannot see extents), outputs are allocated
with torch, and the call is enqueued on torch's current stream of the
tensors' device.  Every step of the operation runs in the HIP library.

Operation and layouts: see include/dcn.h (the DCNv3/DCNv4 sampling core of
wmrh.cn/news/61976 section 二 and pnsm.cn/news/2029644.html section 2).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _capi

_DTYPES = {torch.float32: _capi.DCN_F32, torch.float16: _capi.DCN_F16,
           torch.bfloat16: _capi.DCN_BF16}


def _pair(v) -> Tuple[int, int]:
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def make_problem(x_shape, *, groups, kernel=3, stride=1, pad=1, dilation=1, offset_scale=2.0,
                 softmax=True, dtype=torch.float32, remove_center=False) -> _capi.dcn_problem:
    """The dcn_problem of an (N, H, W, C) input and the operator's arguments."""
    n, h, w, c = (int(v) for v in x_shape)
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    return _capi.make_problem(n=n, h=h, w=w, c=c, groups=int(groups), kernel_h=kh, kernel_w=kw,
                              stride_h=sh, stride_w=sw, pad_h=ph, pad_w=pw, dilation_h=dh,
                              dilation_w=dw, offset_scale=float(offset_scale),
                              softmax=1 if softmax else 0, dtype=_DTYPES[dtype],
                              remove_center=1 if remove_center else 0)


def dcn_check(x_shape, **kw) -> Tuple[int, int]:
    """Validate a problem in the library (host only); returns (Ho, Wo)."""
    st, ho, wo = _capi.dcn_check(make_problem(x_shape, **kw))
    _capi.raise_on(st)
    return ho, wo


def _expect(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _overlaps(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Whether the byte ranges of two tensors intersect."""
    if a.numel() == 0 or b.numel() == 0:
        return False
    a0, b0 = a.data_ptr(), b.data_ptr()
    return a0 < b0 + b.numel() * b.element_size() and b0 < a0 + a.numel() * a.element_size()


def _no_alias(outputs, inputs):
    for oname, o in outputs:
        for iname, i in inputs:
            if _overlaps(o, i):
                raise ValueError(f"{oname} overlaps {iname}: outputs must not alias other tensors")


def _shapes(x: torch.Tensor, groups, kernel, stride, pad, dilation, offset_scale, softmax,
            remove_center=False):
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("input must be a 4-D (N, H, W, C) tensor")
    if x.device.type != "cuda":
        raise ValueError("the DCN core runs on the GPU only: input must be a cuda tensor")
    p = make_problem(x.shape, groups=groups, kernel=kernel, stride=stride, pad=pad,
                     dilation=dilation, offset_scale=offset_scale, softmax=softmax, dtype=x.dtype,
                     remove_center=remove_center)
    st, ho, wo = _capi.dcn_check(p)
    _capi.raise_on(st)
    K = p.kernel_h * p.kernel_w - p.remove_center
    n = x.shape[0]
    return p, {"offset": (n, ho, wo, groups, K, 2), "mask": (n, ho, wo, groups, K),
               "out": (n, ho, wo, x.shape[3])}


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def dcn_forward(x: torch.Tensor, offset: torch.Tensor, mask: torch.Tensor, *, groups: int,
                kernel=3, stride=1, pad=1, dilation=1, offset_scale: float = 2.0,
                softmax: bool = True, remove_center: bool = False,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Forward of the DCN core; returns (N, Ho, Wo, C) in x's dtype."""
    p, shp = _shapes(x, groups, kernel, stride, pad, dilation, offset_scale, softmax, remove_center)
    _expect(x, "input", x.shape, x.dtype, x.device)
    _expect(offset, "offset", shp["offset"], x.dtype, x.device)
    _expect(mask, "mask", shp["mask"], x.dtype, x.device)
    if out is None:
        out = torch.empty(shp["out"], dtype=x.dtype, device=x.device)
    _expect(out, "out", shp["out"], x.dtype, x.device)
    _no_alias([("out", out)], [("input", x), ("offset", offset), ("mask", mask)])
    with torch.cuda.device(x.device):
        st = _capi.dcn_forward(p, x.data_ptr(), offset.data_ptr(), mask.data_ptr(),
                               out.data_ptr(), _stream(x.device))
    _capi.raise_on(st)
    return out


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def dcn_forward_generated(x: torch.Tensor, guide: torch.Tensor, w_offset: torch.Tensor,
                          b_offset: Optional[torch.Tensor], w_mask: torch.Tensor, b_mask: Optional[torch.Tensor],
                          *, groups: int, kernel=3, stride=1, pad=1, dilation=1, offset_scale: float = 2.0,
                          softmax: bool = True, remove_center: bool = False,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Forward with the offsets and mask generated in the kernel from
    ``guide`` (N, Ho, Wo, Cgd) by the linear branches w_offset (G*K*2, Cgd),
    b_offset and w_mask (G*K, Cgd), b_mask (biases may be None)."""
    p, shp = _shapes(x, groups, kernel, stride, pad, dilation, offset_scale, softmax, remove_center)
    n, ho, wo, G, K, _ = shp["offset"]
    if guide.dim() != 4:
        raise ValueError("guide must be a 4-D (N, Ho, Wo, Cgd) tensor")
    cgd = guide.shape[3]
    _expect(x, "input", x.shape, x.dtype, x.device)
    _expect(guide, "guide", (n, ho, wo, cgd), x.dtype, x.device)
    _expect(w_offset, "w_offset", (G * K * 2, cgd), x.dtype, x.device)
    _expect(w_mask, "w_mask", (G * K, cgd), x.dtype, x.device)
    if b_offset is not None:
        _expect(b_offset, "b_offset", (G * K * 2,), x.dtype, x.device)
    if b_mask is not None:
        _expect(b_mask, "b_mask", (G * K,), x.dtype, x.device)
    if out is None:
        out = torch.empty(shp["out"], dtype=x.dtype, device=x.device)
    _expect(out, "out", shp["out"], x.dtype, x.device)
    ins = [("input", x), ("guide", guide), ("w_offset", w_offset), ("w_mask", w_mask)]
    ins += [(k, t) for k, t in (("b_offset", b_offset), ("b_mask", b_mask)) if t is not None]
    _no_alias([("out", out)], ins)
    with torch.cuda.device(x.device):
        st = _capi.dcn_forward_generated(p, cgd, x.data_ptr(), guide.data_ptr(), w_offset.data_ptr(),
                                         _ptr(b_offset), w_mask.data_ptr(), _ptr(b_mask), out.data_ptr(),
                                         _stream(x.device))
    _capi.raise_on(st)
    return out


def dcn_forward_projected(x: torch.Tensor, offset: torch.Tensor, mask: torch.Tensor, w_out: torch.Tensor,
                          b_out: Optional[torch.Tensor], *, groups: int, kernel=3, stride=1, pad=1, dilation=1,
                          offset_scale: float = 2.0, softmax: bool = True, remove_center: bool = False,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Forward followed in the kernel by the output projection w_out (C, C),
    b_out (C) or None."""
    p, shp = _shapes(x, groups, kernel, stride, pad, dilation, offset_scale, softmax, remove_center)
    c = x.shape[3]
    _expect(x, "input", x.shape, x.dtype, x.device)
    _expect(offset, "offset", shp["offset"], x.dtype, x.device)
    _expect(mask, "mask", shp["mask"], x.dtype, x.device)
    _expect(w_out, "w_out", (c, c), x.dtype, x.device)
    if b_out is not None:
        _expect(b_out, "b_out", (c,), x.dtype, x.device)
    if out is None:
        out = torch.empty(shp["out"], dtype=x.dtype, device=x.device)
    _expect(out, "out", shp["out"], x.dtype, x.device)
    ins = [("input", x), ("offset", offset), ("mask", mask), ("w_out", w_out)]
    if b_out is not None:
        ins.append(("b_out", b_out))
    _no_alias([("out", out)], ins)
    with torch.cuda.device(x.device):
        st = _capi.dcn_forward_projected(p, x.data_ptr(), offset.data_ptr(), mask.data_ptr(), w_out.data_ptr(),
                                         _ptr(b_out), out.data_ptr(), _stream(x.device))
    _capi.raise_on(st)
    return out


def _backward_args(x, offset, mask, grad_out, groups, kernel, stride, pad, dilation, offset_scale, softmax,
                   remove_center, grad_input, grad_offset, grad_mask):
    """Checked problem and gradient tensors of a backward call (allocated
    here when not given)."""
    p, shp = _shapes(x, groups, kernel, stride, pad, dilation, offset_scale, softmax, remove_center)
    _expect(x, "input", x.shape, x.dtype, x.device)
    _expect(offset, "offset", shp["offset"], x.dtype, x.device)
    _expect(mask, "mask", shp["mask"], x.dtype, x.device)
    _expect(grad_out, "grad_out", shp["out"], x.dtype, x.device)
    if grad_input is None:
        grad_input = torch.empty_like(x)
    if grad_offset is None:
        grad_offset = torch.empty_like(offset)
    if grad_mask is None:
        grad_mask = torch.empty_like(mask)
    _expect(grad_input, "grad_input", x.shape, x.dtype, x.device)
    _expect(grad_offset, "grad_offset", shp["offset"], x.dtype, x.device)
    _expect(grad_mask, "grad_mask", shp["mask"], x.dtype, x.device)
    outs = [("grad_input", grad_input), ("grad_offset", grad_offset), ("grad_mask", grad_mask)]
    _no_alias(outs, [("input", x), ("offset", offset), ("mask", mask), ("grad_out", grad_out)])
    for k, (a, ta) in enumerate(outs):
        _no_alias([(a, ta)], outs[k + 1:])
    return p, outs


def dcn_backward(x: torch.Tensor, offset: torch.Tensor, mask: torch.Tensor,
                 grad_out: torch.Tensor, *, groups: int, kernel=3, stride=1, pad=1, dilation=1,
                 offset_scale: float = 2.0, softmax: bool = True, remove_center: bool = False,
                 grad_input: Optional[torch.Tensor] = None,
                 grad_offset: Optional[torch.Tensor] = None,
                 grad_mask: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None):
    """Backward of the DCN core; returns (grad_input, grad_offset, grad_mask).

    16-bit I/O accumulates grad_input in an fp32 device workspace
    (``backward_workspace_bytes``); pass a ``workspace`` tensor on x's device
    to reuse one, else a fresh one is taken from torch's allocator."""
    p, outs = _backward_args(x, offset, mask, grad_out, groups, kernel, stride, pad, dilation, offset_scale,
                             softmax, remove_center, grad_input, grad_offset, grad_mask)
    grad_input, grad_offset, grad_mask = (t for _, t in outs)
    st, ws_bytes = _capi.dcn_backward_workspace_size(p)
    _capi.raise_on(st)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    ws_ptr, ws_have = None, 0
    if workspace is not None:
        if workspace.device != x.device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {x.device}")
        _no_alias([("workspace", workspace)], outs + [("input", x), ("offset", offset), ("mask", mask),
                                                       ("grad_out", grad_out)])
        ws_ptr, ws_have = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(x.device):
        st = _capi.dcn_backward(p, x.data_ptr(), offset.data_ptr(), mask.data_ptr(),
                                grad_out.data_ptr(), grad_input.data_ptr(),
                                grad_offset.data_ptr(), grad_mask.data_ptr(), ws_ptr, ws_have,
                                _stream(x.device))
    _capi.raise_on(st)
    return grad_input, grad_offset, grad_mask


def dcn_backward_noalloc(x: torch.Tensor, offset: torch.Tensor, mask: torch.Tensor,
                         grad_out: torch.Tensor, *, groups: int, kernel=3, stride=1, pad=1, dilation=1,
                         offset_scale: float = 2.0, softmax: bool = True, remove_center: bool = False,
                         grad_input: Optional[torch.Tensor] = None,
                         grad_offset: Optional[torch.Tensor] = None,
                         grad_mask: Optional[torch.Tensor] = None):
    """dcn_backward through the library's allocation-free entry point: 16-bit
    I/O accumulates in the library's fixed per-GPU scratch instead of a
    workspace.  With the gradient tensors passed in, the call allocates no
    device memory; 16-bit calls on one GPU must not overlap."""
    p, outs = _backward_args(x, offset, mask, grad_out, groups, kernel, stride, pad, dilation, offset_scale,
                             softmax, remove_center, grad_input, grad_offset, grad_mask)
    grad_input, grad_offset, grad_mask = (t for _, t in outs)
    with torch.cuda.device(x.device):
        st = _capi.dcn_backward_noalloc(p, x.data_ptr(), offset.data_ptr(), mask.data_ptr(),
                                        grad_out.data_ptr(), grad_input.data_ptr(),
                                        grad_offset.data_ptr(), grad_mask.data_ptr(), _stream(x.device))
    _capi.raise_on(st)
    return grad_input, grad_offset, grad_mask


def backward_workspace_bytes(x: torch.Tensor, *, groups: int, kernel=3, stride=1, pad=1, dilation=1,
                             offset_scale: float = 2.0, softmax: bool = True,
                             remove_center: bool = False) -> int:
    """Device workspace bytes that dcn_backward needs for this problem (0 for fp32)."""
    p, _ = _shapes(x, groups, kernel, stride, pad, dilation, offset_scale, softmax, remove_center)
    st, n = _capi.dcn_backward_workspace_size(p)
    _capi.raise_on(st)
    return n


class DCNCore(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in the HIP library."""

    @staticmethod
    def forward(ctx, x, offset, mask, groups, kernel, stride, pad, dilation, offset_scale, softmax,
                remove_center):
        x, offset, mask = x.contiguous(), offset.contiguous(), mask.contiguous()
        ctx.save_for_backward(x, offset, mask)
        ctx.args = dict(groups=groups, kernel=kernel, stride=stride, pad=pad, dilation=dilation,
                        offset_scale=offset_scale, softmax=softmax, remove_center=remove_center)
        return dcn_forward(x, offset, mask, **ctx.args)

    @staticmethod
    def backward(ctx, grad_out):
        x, offset, mask = ctx.saved_tensors
        gx, goff, gm = dcn_backward(x, offset, mask, grad_out.contiguous(), **ctx.args)
        return gx, goff, gm, None, None, None, None, None, None, None, None


def dcn_core(x, offset, mask, *, groups, kernel=3, stride=1, pad=1, dilation=1,
             offset_scale=2.0, softmax=True, remove_center=False):
    """Differentiable DCN core (forward and backward in the HIP library, fp32
    or 16-bit I/O)."""
    return DCNCore.apply(x, offset, mask, groups, kernel, stride, pad, dilation, offset_scale,
                         softmax, remove_center)
