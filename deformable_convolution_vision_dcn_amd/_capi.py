"""ctypes view of the C ABI in include/dcn.h (libdcn_mi355x.so).

Argument marshalling only.  The library must have been built
(``__graft_entry__.build()`` or ``python deformable_convolution_vision_dcn_amd/build.py``);
there is no fallback implementation, so a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import pathlib

LIB_PATH = pathlib.Path(os.environ.get(
    "DCN_MI355X_LIB", pathlib.Path(__file__).resolve().parent / "libdcn_mi355x.so"))

ABI_VERSION = 6

# bytes of the library's fixed scratch behind dcn_backward_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20

DCN_F32, DCN_F16, DCN_BF16 = 0, 1, 2

STATUS = {
    0: "DCN_OK",
    -1: "DCN_ERR_NULL",
    -2: "DCN_ERR_SHAPE",
    -3: "DCN_ERR_UNSUPPORTED",
    -4: "DCN_ERR_ALIGN",
    -5: "DCN_ERR_TOO_LARGE",
    -6: "DCN_ERR_HIP",
    -7: "DCN_ERR_ABI",
    -8: "DCN_ERR_ARG",
    -9: "DCN_ERR_WORKSPACE",
    -10: "DCN_ERR_SCRATCH",
}
CODES = {v: k for k, v in STATUS.items()}


class dcn_problem(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("n", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32),
        ("c", ctypes.c_int32), ("groups", ctypes.c_int32),
        ("kernel_h", ctypes.c_int32), ("kernel_w", ctypes.c_int32),
        ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
        ("pad_h", ctypes.c_int32), ("pad_w", ctypes.c_int32),
        ("dilation_h", ctypes.c_int32), ("dilation_w", ctypes.c_int32),
        ("offset_scale", ctypes.c_float),
        ("softmax", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("remove_center", ctypes.c_int32),
    ]


def make_problem(**kw) -> dcn_problem:
    p = dcn_problem()
    p.struct_size = ctypes.sizeof(dcn_problem)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


class DCNError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class LibraryMissing(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once per process)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise LibraryMissing(
                f"{LIB_PATH} is not built: run __graft_entry__.build() "
                "(the DCN core has no fallback implementation)")
        L = ctypes.CDLL(str(LIB_PATH))
        P = ctypes.POINTER(dcn_problem)
        vp = ctypes.c_void_p
        L.dcn_abi_version.restype = ctypes.c_int
        L.dcn_abi_version.argtypes = []
        L.dcn_check.restype = ctypes.c_int
        L.dcn_check.argtypes = [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        L.dcn_forward.restype = ctypes.c_int
        L.dcn_forward.argtypes = [P, vp, vp, vp, vp, vp]
        L.dcn_backward.restype = ctypes.c_int
        L.dcn_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
        L.dcn_forward_generated.restype = ctypes.c_int
        L.dcn_forward_generated.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.dcn_forward_projected.restype = ctypes.c_int
        L.dcn_forward_projected.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.dcn_backward_noalloc.restype = ctypes.c_int
        L.dcn_backward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.dcn_backward_workspace_size.restype = ctypes.c_int
        L.dcn_backward_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_uint64)]
        L.dcn_status_string.restype = ctypes.c_char_p
        L.dcn_status_string.argtypes = [ctypes.c_int]
        if L.dcn_abi_version() != ABI_VERSION:
            raise LibraryMissing(f"{LIB_PATH}: ABI version {L.dcn_abi_version()} != {ABI_VERSION}")
        _lib = L
    return _lib


def dcn_abi_version() -> int:
    return lib().dcn_abi_version()


def dcn_status_string(status: int) -> str:
    return lib().dcn_status_string(status).decode()


def dcn_check(p: dcn_problem):
    """Returns (status, ho, wo)."""
    ho = ctypes.c_int64(0)
    wo = ctypes.c_int64(0)
    st = lib().dcn_check(ctypes.byref(p), ctypes.byref(ho), ctypes.byref(wo))
    return st, ho.value, wo.value


def dcn_forward(p: dcn_problem, input_ptr, offset_ptr, mask_ptr, output_ptr, stream) -> int:
    return lib().dcn_forward(ctypes.byref(p), input_ptr, offset_ptr, mask_ptr, output_ptr, stream)


def dcn_forward_generated(p: dcn_problem, guide_channels, input_ptr, guide_ptr, w_offset_ptr, b_offset_ptr,
                          w_mask_ptr, b_mask_ptr, output_ptr, stream) -> int:
    return lib().dcn_forward_generated(ctypes.byref(p), guide_channels, input_ptr, guide_ptr, w_offset_ptr,
                                       b_offset_ptr, w_mask_ptr, b_mask_ptr, output_ptr, stream)


def dcn_forward_projected(p: dcn_problem, input_ptr, offset_ptr, mask_ptr, w_out_ptr, b_out_ptr, output_ptr,
                          stream) -> int:
    return lib().dcn_forward_projected(ctypes.byref(p), input_ptr, offset_ptr, mask_ptr, w_out_ptr, b_out_ptr,
                                       output_ptr, stream)


def dcn_backward_workspace_size(p: dcn_problem):
    """Returns (status, bytes)."""
    n = ctypes.c_uint64(0)
    st = lib().dcn_backward_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def dcn_backward(p: dcn_problem, input_ptr, offset_ptr, mask_ptr, grad_out_ptr, grad_in_ptr,
                 grad_offset_ptr, grad_mask_ptr, workspace_ptr, workspace_bytes, stream) -> int:
    return lib().dcn_backward(ctypes.byref(p), input_ptr, offset_ptr, mask_ptr, grad_out_ptr,
                              grad_in_ptr, grad_offset_ptr, grad_mask_ptr, workspace_ptr,
                              workspace_bytes, stream)


def dcn_backward_noalloc(p: dcn_problem, input_ptr, offset_ptr, mask_ptr, grad_out_ptr, grad_in_ptr,
                         grad_offset_ptr, grad_mask_ptr, stream) -> int:
    return lib().dcn_backward_noalloc(ctypes.byref(p), input_ptr, offset_ptr, mask_ptr, grad_out_ptr,
                                      grad_in_ptr, grad_offset_ptr, grad_mask_ptr, stream)


def raise_on(status: int) -> None:
    if status != 0:
        raise DCNError(status, dcn_status_string(status))
