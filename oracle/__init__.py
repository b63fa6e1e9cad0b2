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
