"""fp64 CPU oracle for the DCN core -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does, and shares no code with it.

The arithmetic lives in ``dcn_oracle.c`` (plain loops over the definition, in
fp64); this module only marshals numpy arrays to it.  Arrays of any float dtype
(float16, float32, float64, or bfloat16 values already widened by the caller)
are converted exactly to float64 before the call.

Layouts (the pages' NHWC convention, pnsm.cn/news/2029644.html section 2.3):
  x      (N, H, W, C)                  C = groups * Cg
  offset (N, Ho, Wo, G, K, 2)          pair stored as (x, y)
  mask   (N, Ho, Wo, G, K)             logits (softmax=True) or raw weights
  y      (N, Ho, Wo, C)
K = KH*KW points, or KH*KW - 1 with remove_center=True (odd KH and KW; the
centre point is dropped, pnsm.cn/news/2029644.html section 3.3).

Beside the core: ``linear`` (a linear layer), ``forward_om`` (the core with
its offsets and mask generated from a guide feature by two linear branches,
wmrh.cn/news/61976 section 二 steps 2-3) and ``forward_proj`` (the core
followed by the output_proj linear layer, step 4).

Every function here is pinned by ``tests/test_oracle_pins.py``; no function is
parity-unpinned.
"""
from __future__ import annotations

import ctypes
import pathlib

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
LIB_PATH = _HERE / "libdcn_oracle.so"
SOURCE_PATH = _HERE / "dcn_oracle.c"


class _RefProblem(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64), ("h", ctypes.c_int64), ("w", ctypes.c_int64),
        ("c", ctypes.c_int64), ("groups", ctypes.c_int64),
        ("kh", ctypes.c_int64), ("kw", ctypes.c_int64),
        ("stride_h", ctypes.c_int64), ("stride_w", ctypes.c_int64),
        ("pad_h", ctypes.c_int64), ("pad_w", ctypes.c_int64),
        ("dil_h", ctypes.c_int64), ("dil_w", ctypes.c_int64),
        ("offset_scale", ctypes.c_double),
        ("softmax", ctypes.c_int64),
        ("remove_center", ctypes.c_int64),
    ]


def _pair(v):
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """One loaded build of the oracle library (the default build, or a test's
    deliberately mutated copy)."""

    def __init__(self, lib_path=LIB_PATH):
        lib_path = pathlib.Path(lib_path)
        if not lib_path.exists():
            from .build import build
            build()
        lib = ctypes.CDLL(str(lib_path))
        P = ctypes.POINTER(_RefProblem)
        D = ctypes.POINTER(ctypes.c_double)
        I = ctypes.POINTER(ctypes.c_int64)
        lib.ref_out_size.restype = ctypes.c_int64
        lib.ref_out_size.argtypes = [ctypes.c_int64] * 5
        lib.ref_forward.restype = None
        lib.ref_forward.argtypes = [P, D, D, D, D]
        lib.ref_forward_pixels.restype = None
        lib.ref_forward_pixels.argtypes = [P, D, D, D, I, ctypes.c_int64, D]
        lib.ref_backward.restype = None
        lib.ref_backward.argtypes = [P, D, D, D, D, D, D, D]
        i64 = ctypes.c_int64
        lib.ref_linear.restype = None
        lib.ref_linear.argtypes = [i64, i64, i64, D, D, D, D]
        lib.ref_forward_om.restype = None
        lib.ref_forward_om.argtypes = [P, D, D, i64, D, D, D, D, D]
        lib.ref_forward_proj.restype = None
        lib.ref_forward_proj.argtypes = [P, D, D, D, D, D, D]
        self._lib = lib

    def out_size(self, in_size, kernel, stride, pad, dilation):
        """Output extent along one axis: floor((in + 2p - d(k-1) - 1)/s) + 1."""
        return int(self._lib.ref_out_size(in_size, kernel, stride, pad, dilation))

    def _problem(self, x_shape, groups, kernel, stride, pad, dilation, offset_scale, softmax,
                 remove_center=False):
        n, h, w, c = (int(v) for v in x_shape)
        kh, kw = _pair(kernel)
        if remove_center and (kh % 2 == 0 or kw % 2 == 0 or kh * kw < 2):
            raise ValueError("remove_center needs odd kernel sizes and at least 3 points")
        sh, sw = _pair(stride)
        ph, pw = _pair(pad)
        dh, dw = _pair(dilation)
        if groups <= 0 or c % groups:
            raise ValueError("C must be a multiple of groups")
        p = _RefProblem(n, h, w, c, groups, kh, kw, sh, sw, ph, pw, dh, dw,
                        float(offset_scale), 1 if softmax else 0, 1 if remove_center else 0)
        ho = self.out_size(h, kh, sh, ph, dh)
        wo = self.out_size(w, kw, sw, pw, dw)
        return p, ho, wo, kh * kw - (1 if remove_center else 0)

    @staticmethod
    def _check_shapes(x, offset, mask, groups, ho, wo, K):
        n = x.shape[0]
        if offset.shape != (n, ho, wo, groups, K, 2):
            raise ValueError(f"offset shape {offset.shape} != {(n, ho, wo, groups, K, 2)}")
        if mask.shape != (n, ho, wo, groups, K):
            raise ValueError(f"mask shape {mask.shape} != {(n, ho, wo, groups, K)}")

    def forward(self, x, offset, mask, *, groups, kernel=3, stride=1, pad=1, dilation=1,
                offset_scale=2.0, softmax=True, remove_center=False):
        """Full fp64 forward; returns y (N, Ho, Wo, C) as float64."""
        x, offset, mask = _f64(x), _f64(offset), _f64(mask)
        p, ho, wo, K = self._problem(x.shape, groups, kernel, stride, pad, dilation,
                                     offset_scale, softmax, remove_center)
        self._check_shapes(x, offset, mask, groups, ho, wo, K)
        y = np.zeros((x.shape[0], ho, wo, x.shape[3]), dtype=np.float64)
        self._lib.ref_forward(ctypes.byref(p), _dptr(x), _dptr(offset), _dptr(mask), _dptr(y))
        return y

    def forward_pixels(self, x, offset, mask, pixels, *, groups, kernel=3, stride=1, pad=1,
                       dilation=1, offset_scale=2.0, softmax=True, remove_center=False):
        """fp64 forward at selected output pixels.

        ``pixels`` holds flat indices (n*Ho + ho)*Wo + wo; returns (len(pixels), C).
        """
        x, offset, mask = _f64(x), _f64(offset), _f64(mask)
        p, ho, wo, K = self._problem(x.shape, groups, kernel, stride, pad, dilation,
                                     offset_scale, softmax, remove_center)
        self._check_shapes(x, offset, mask, groups, ho, wo, K)
        pix = np.ascontiguousarray(pixels, dtype=np.int64).reshape(-1)
        if pix.size and (pix.min() < 0 or pix.max() >= x.shape[0] * ho * wo):
            raise ValueError("pixel index out of range")
        y = np.zeros((pix.size, x.shape[3]), dtype=np.float64)
        self._lib.ref_forward_pixels(ctypes.byref(p), _dptr(x), _dptr(offset), _dptr(mask),
                                     pix.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     pix.size, _dptr(y))
        return y

    def backward(self, x, offset, mask, grad_out, *, groups, kernel=3, stride=1, pad=1,
                 dilation=1, offset_scale=2.0, softmax=True, remove_center=False):
        """fp64 backward; returns (grad_input, grad_offset, grad_mask) as float64.

        grad_mask is taken with respect to the tensor passed as ``mask`` (the
        logits when softmax=True).
        """
        x, offset, mask, gy = _f64(x), _f64(offset), _f64(mask), _f64(grad_out)
        p, ho, wo, K = self._problem(x.shape, groups, kernel, stride, pad, dilation,
                                     offset_scale, softmax, remove_center)
        self._check_shapes(x, offset, mask, groups, ho, wo, K)
        if gy.shape != (x.shape[0], ho, wo, x.shape[3]):
            raise ValueError("grad_out shape mismatch")
        gx = np.zeros_like(x)
        goff = np.zeros_like(offset)
        gmask = np.zeros_like(mask)
        self._lib.ref_backward(ctypes.byref(p), _dptr(x), _dptr(offset), _dptr(mask),
                               _dptr(gy), _dptr(gx), _dptr(goff), _dptr(gmask))
        return gx, goff, gmask


    def linear(self, x, w, b=None):
        """fp64 linear layer over the last axis: x (..., nin), w (nout, nin),
        b (nout) or None; returns (..., nout)."""
        x, w = _f64(x), _f64(w)
        nin = x.shape[-1]
        if w.ndim != 2 or w.shape[1] != nin:
            raise ValueError(f"weight shape {w.shape} does not match {nin} input features")
        nout = w.shape[0]
        bb = None if b is None else _f64(b)
        if bb is not None and bb.shape != (nout,):
            raise ValueError("bias shape mismatch")
        rows = x.size // nin if nin else 0
        out = np.zeros(x.shape[:-1] + (nout,), dtype=np.float64)
        self._lib.ref_linear(rows, nin, nout, _dptr(x), _dptr(w), None if bb is None else _dptr(bb), _dptr(out))
        return out

    def forward_om(self, x, guide, w_offset, b_offset, w_mask, b_mask, *, groups, kernel=3, stride=1,
                   pad=1, dilation=1, offset_scale=2.0, softmax=True, remove_center=False):
        """fp64 forward with the offsets and mask generated from ``guide``
        (N, Ho, Wo, Cgd) by the linear branches w_offset (G*K*2, Cgd),
        b_offset and w_mask (G*K, Cgd), b_mask (biases may be None)."""
        x, guide, wo_, wm = _f64(x), _f64(guide), _f64(w_offset), _f64(w_mask)
        p, ho, wo, K = self._problem(x.shape, groups, kernel, stride, pad, dilation,
                                     offset_scale, softmax, remove_center)
        n, cgd = x.shape[0], guide.shape[-1]
        if guide.shape != (n, ho, wo, cgd):
            raise ValueError(f"guide shape {guide.shape} != {(n, ho, wo, cgd)}")
        if wo_.shape != (groups * K * 2, cgd) or wm.shape != (groups * K, cgd):
            raise ValueError("generation weight shapes do not match")
        bo = None if b_offset is None else _f64(b_offset)
        bm = None if b_mask is None else _f64(b_mask)
        if (bo is not None and bo.shape != (groups * K * 2,)) or (bm is not None and bm.shape != (groups * K,)):
            raise ValueError("generation bias shapes do not match")
        y = np.zeros((n, ho, wo, x.shape[3]), dtype=np.float64)
        self._lib.ref_forward_om(ctypes.byref(p), _dptr(x), _dptr(guide), cgd, _dptr(wo_),
                                 None if bo is None else _dptr(bo), _dptr(wm),
                                 None if bm is None else _dptr(bm), _dptr(y))
        return y

    def forward_proj(self, x, offset, mask, w_out, b_out, *, groups, kernel=3, stride=1, pad=1,
                     dilation=1, offset_scale=2.0, softmax=True, remove_center=False):
        """fp64 forward followed by the output projection w_out (C, C), b_out
        (C) or None."""
        x, offset, mask, w = _f64(x), _f64(offset), _f64(mask), _f64(w_out)
        p, ho, wo, K = self._problem(x.shape, groups, kernel, stride, pad, dilation,
                                     offset_scale, softmax, remove_center)
        self._check_shapes(x, offset, mask, groups, ho, wo, K)
        c = x.shape[3]
        if w.shape != (c, c):
            raise ValueError(f"w_out shape {w.shape} != {(c, c)}")
        b = None if b_out is None else _f64(b_out)
        if b is not None and b.shape != (c,):
            raise ValueError("b_out shape mismatch")
        out = np.zeros((x.shape[0], ho, wo, c), dtype=np.float64)
        self._lib.ref_forward_proj(ctypes.byref(p), _dptr(x), _dptr(offset), _dptr(mask), _dptr(w),
                                   None if b is None else _dptr(b), _dptr(out))
        return out


_default = None


def default() -> Oracle:
    """The oracle built from ``dcn_oracle.c`` as committed."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def out_size(in_size, kernel, stride, pad, dilation):
    return default().out_size(in_size, kernel, stride, pad, dilation)


def out_hw(wl):
    """(Ho, Wo) of a synth.Workload from the oracle's own output-size rule."""
    return (out_size(wl.h, wl.kernel[0], wl.stride[0], wl.pad[0], wl.dilation[0]),
            out_size(wl.w, wl.kernel[1], wl.stride[1], wl.pad[1], wl.dilation[1]))


def forward(*args, **kwargs):
    return default().forward(*args, **kwargs)


def forward_pixels(*args, **kwargs):
    return default().forward_pixels(*args, **kwargs)


def backward(*args, **kwargs):
    return default().backward(*args, **kwargs)


def linear(*args, **kwargs):
    return default().linear(*args, **kwargs)


def forward_om(*args, **kwargs):
    return default().forward_om(*args, **kwargs)


def forward_proj(*args, **kwargs):
    return default().forward_proj(*args, **kwargs)
