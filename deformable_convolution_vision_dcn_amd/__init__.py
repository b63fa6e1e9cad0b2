"""MI355X-native (gfx950) DCNv3/DCNv4 deformable-sampling core.

The operation runs in hand-written HIP kernels behind the C ABI of
include/dcn.h (libdcn_mi355x.so); this package is its thin Python binding.
"""
from ._capi import DCNError, LibraryMissing, dcn_abi_version, dcn_status_string  # noqa: F401
from .ops import (backward_workspace_bytes, dcn_backward, dcn_backward_noalloc, dcn_check, dcn_core,  # noqa: F401
                  dcn_forward, dcn_forward_generated, dcn_forward_projected, make_problem)

__all__ = ["dcn_forward", "dcn_forward_generated", "dcn_forward_projected", "dcn_backward", "dcn_backward_noalloc", "backward_workspace_bytes", "dcn_check", "dcn_core", "dcn_status_string",
           "dcn_abi_version", "make_problem", "DCNError", "LibraryMissing"]
