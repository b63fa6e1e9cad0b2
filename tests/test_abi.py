"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and its host-side validation (dcn_check and the argument checks
that precede any device call) behaves as documented.  No compute calls."""
import ctypes
import pathlib
import re
import subprocess

import pytest

import oracle
from deformable_convolution_vision_dcn_amd import _capi

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "dcn.h"


@pytest.fixture(scope="module")
def lib():
    if not _capi.LIB_PATH.exists():
        from deformable_convolution_vision_dcn_amd.build import build
        build()
    return _capi.lib()


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dcn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["dcn_abi_version", "dcn_backward", "dcn_backward_noalloc",
                                    "dcn_backward_workspace_size", "dcn_check", "dcn_forward",
                                    "dcn_forward_generated", "dcn_forward_projected", "dcn_status_string"]


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(_capi.LIB_PATH)], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, f"{name} not exported"
        assert hasattr(lib, name)


def test_abi_version_matches_header(lib):
    m = re.search(r"#define DCN_ABI_VERSION (\d+)", HEADER.read_text())
    assert lib.dcn_abi_version() == int(m.group(1)) == _capi.ABI_VERSION


def test_status_codes_match_header():
    text = HEADER.read_text()
    for name, code in re.findall(r"(DCN_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", text):
        assert _capi.CODES[name] == int(code)
    assert len(_capi.CODES) == len(re.findall(r"(DCN_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", text))


def test_problem_struct_layout_is_guarded(lib):
    # 18 four-byte fields, no padding
    assert ctypes.sizeof(_capi.dcn_problem) == 72
    p = _capi.make_problem(n=1, h=8, w=8, c=16, groups=1, kernel_h=3, kernel_w=3, stride_h=1,
                           stride_w=1, pad_h=1, pad_w=1, dilation_h=1, dilation_w=1,
                           offset_scale=2.0, softmax=1, dtype=0)
    assert _capi.dcn_check(p)[0] == 0
    p.struct_size = 68  # the layout before remove_center
    assert _capi.dcn_check(p)[0] == _capi.CODES["DCN_ERR_ABI"]


def test_status_strings(lib):
    for code in _capi.STATUS:
        s = _capi.dcn_status_string(code)
        assert isinstance(s, str) and s
    assert _capi.dcn_status_string(-99) == "unknown status"


BASE = dict(n=2, h=9, w=7, c=32, groups=2, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1,
            pad_h=1, pad_w=1, dilation_h=1, dilation_w=1, offset_scale=2.0, softmax=1, dtype=0)


@pytest.mark.parametrize("change,code", [
    ({}, "DCN_OK"),
    ({"n": 0}, "DCN_OK"),
    ({"n": -1}, "DCN_ERR_SHAPE"),
    ({"h": 0}, "DCN_ERR_SHAPE"),
    ({"w": -3}, "DCN_ERR_SHAPE"),
    ({"c": 0}, "DCN_ERR_SHAPE"),
    ({"groups": 0}, "DCN_ERR_SHAPE"),
    ({"groups": 3}, "DCN_ERR_SHAPE"),          # 32 % 3 != 0
    ({"kernel_h": 0}, "DCN_ERR_SHAPE"),
    ({"stride_w": 0}, "DCN_ERR_SHAPE"),
    ({"dilation_h": 0}, "DCN_ERR_SHAPE"),
    ({"pad_w": -1}, "DCN_ERR_SHAPE"),
    ({"h": 2, "pad_h": 0}, "DCN_ERR_SHAPE"),   # 3x3 window does not fit: Ho < 1
    ({"softmax": 2}, "DCN_ERR_ARG"),
    ({"offset_scale": float("nan")}, "DCN_ERR_ARG"),
    ({"offset_scale": float("inf")}, "DCN_ERR_ARG"),
    ({"dtype": 3}, "DCN_ERR_UNSUPPORTED"),
    ({"groups": 4}, "DCN_ERR_UNSUPPORTED"),    # 8 channels per group
    ({"groups": 1}, "DCN_ERR_UNSUPPORTED"),    # 32 channels per group
    ({"kernel_h": 9, "kernel_w": 9, "pad_h": 4, "pad_w": 4}, "DCN_ERR_UNSUPPORTED"),  # 81 points
    ({"h": 1 << 25}, "DCN_ERR_TOO_LARGE"),
    ({"h": 8192, "w": 8192, "c": 32}, "DCN_ERR_TOO_LARGE"),   # 8 GiB per image
    # 2048x2048x64 fp32: input and output 1 GiB per image; the offsets of a
    # 3x3 window take 1.2 GiB, those of a 5x5 window 3.1 GiB.
    ({"h": 2048, "w": 2048, "c": 64, "groups": 4}, "DCN_OK"),
    ({"h": 2048, "w": 2048, "c": 64, "groups": 4, "kernel_h": 5, "kernel_w": 5,
      "pad_h": 2, "pad_w": 2}, "DCN_ERR_TOO_LARGE"),
    # remove_center: a 0/1 flag, odd kernel sizes only, at least one point left
    ({"remove_center": 1}, "DCN_OK"),
    ({"remove_center": 1, "kernel_h": 5, "kernel_w": 3, "pad_h": 2}, "DCN_OK"),
    ({"remove_center": 2}, "DCN_ERR_ARG"),
    ({"remove_center": -1}, "DCN_ERR_ARG"),
    ({"remove_center": 1, "kernel_h": 4, "pad_h": 2}, "DCN_ERR_ARG"),
    ({"remove_center": 1, "kernel_h": 1, "kernel_w": 1, "pad_h": 0, "pad_w": 0}, "DCN_ERR_SHAPE"),
    # 65 grid points less the centre is 64: within the limit
    ({"remove_center": 1, "kernel_h": 5, "kernel_w": 13, "pad_h": 2, "pad_w": 6, "w": 13}, "DCN_OK"),
    ({"kernel_h": 5, "kernel_w": 13, "pad_h": 2, "pad_w": 6, "w": 13}, "DCN_ERR_UNSUPPORTED"),
])
def test_check_table(lib, change, code):
    p = _capi.make_problem(**{**BASE, **change})
    assert _capi.STATUS[_capi.dcn_check(p)[0]] == code


@pytest.mark.parametrize("geom", [
    dict(h=96, w=96, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1, dilation_h=1, dilation_w=1),
    dict(h=9, w=12, kernel_h=3, kernel_w=3, stride_h=2, stride_w=2, pad_h=0, pad_w=1, dilation_h=1, dilation_w=2),
    dict(h=10, w=7, kernel_h=5, kernel_w=3, stride_h=3, stride_w=1, pad_h=2, pad_w=0, dilation_h=2, dilation_w=1),
    dict(h=1, w=1, kernel_h=1, kernel_w=1, stride_h=1, stride_w=1, pad_h=0, pad_w=0, dilation_h=1, dilation_w=1),
])
def test_check_output_extent_matches_oracle(lib, geom):
    p = _capi.make_problem(**{**BASE, **geom})
    st, ho, wo = _capi.dcn_check(p)
    assert st == 0
    assert ho == oracle.out_size(geom["h"], geom["kernel_h"], geom["stride_h"], geom["pad_h"], geom["dilation_h"])
    assert wo == oracle.out_size(geom["w"], geom["kernel_w"], geom["stride_w"], geom["pad_w"], geom["dilation_w"])


def test_null_problem(lib):
    assert lib.dcn_check(None, None, None) == _capi.CODES["DCN_ERR_NULL"]
    assert lib.dcn_forward(None, None, None, None, None, None) == _capi.CODES["DCN_ERR_NULL"]


def test_argument_checks_before_any_device_call(lib):
    """Null, misaligned and unsupported arguments are refused on the host; the
    fake pointers used here are never dereferenced."""
    p = _capi.make_problem(**BASE)
    F = _capi.dcn_forward
    B = _capi.dcn_backward
    a = 0x10000  # 16-byte aligned, never touched
    assert F(p, None, a, a, a, None) == _capi.CODES["DCN_ERR_NULL"]
    assert F(p, a, a, a, None, None) == _capi.CODES["DCN_ERR_NULL"]
    assert F(p, a + 4, a, a, a, None) == _capi.CODES["DCN_ERR_ALIGN"]
    assert F(p, a, a, a, a + 8, None) == _capi.CODES["DCN_ERR_ALIGN"]
    assert B(p, a, a, a, a, a, a, None, None, 0, None) == _capi.CODES["DCN_ERR_NULL"]
    assert B(p, a, a, a, a, a, a + 2, a, None, 0, None) == _capi.CODES["DCN_ERR_ALIGN"]
    p16 = _capi.make_problem(**{**BASE, "dtype": _capi.DCN_BF16})
    st, need = _capi.dcn_backward_workspace_size(p16)
    assert st == 0 and need == BASE["n"] * BASE["h"] * BASE["w"] * BASE["c"] * 4
    # 16-bit backward at any stride, dilation and point count: the same workspace
    for change in ({"stride_h": 2}, {"dilation_w": 2, "pad_w": 2},
                   {"kernel_h": 5, "kernel_w": 5, "pad_h": 2, "pad_w": 2}):
        for dt in (_capi.DCN_BF16, _capi.DCN_F16):
            p16c = _capi.make_problem(**{**BASE, **change, "dtype": dt})
            assert _capi.dcn_backward_workspace_size(p16c) == (0, need), change
            assert B(p16c, a, a, a, a, a, a, a, a, need - 16, None) == _capi.CODES["DCN_ERR_WORKSPACE"], change
    assert B(p16, a, a, a, a, a, a, None, a, need, None) == _capi.CODES["DCN_ERR_NULL"]
    assert B(p16, a, a, a, a, a, a, a, None, need, None) == _capi.CODES["DCN_ERR_NULL"]
    assert B(p16, a, a, a, a, a, a, a, a + 8, need, None) == _capi.CODES["DCN_ERR_ALIGN"]
    assert B(p16, a, a, a, a, a, a, a, a, need - 16, None) == _capi.CODES["DCN_ERR_WORKSPACE"]
    assert lib.dcn_backward_workspace_size(ctypes.byref(p16), None) == _capi.CODES["DCN_ERR_NULL"]
    # fp32 needs no workspace
    assert _capi.dcn_backward_workspace_size(p) == (0, 0)
    # remove_center: the same workspace rule
    prc = _capi.make_problem(**{**BASE, "remove_center": 1})
    assert _capi.dcn_backward_workspace_size(prc) == (0, 0)
    prc16 = _capi.make_problem(**{**BASE, "remove_center": 1, "dtype": _capi.DCN_F16})
    assert _capi.dcn_backward_workspace_size(prc16) == (0, need)
    prc16s = _capi.make_problem(**{**BASE, "remove_center": 1, "dtype": _capi.DCN_F16, "stride_w": 2})
    assert _capi.dcn_backward_workspace_size(prc16s)[0] == 0
    # dilation 2 on both axes: supported in 16-bit
    pd16 = _capi.make_problem(**{**BASE, "dtype": _capi.DCN_BF16, "dilation_h": 2, "dilation_w": 2,
                                 "pad_h": 2, "pad_w": 2})
    assert _capi.dcn_backward_workspace_size(pd16) == (0, need)
    # N = 0: valid, nothing enqueued, pointers may be NULL
    p0 = _capi.make_problem(**{**BASE, "n": 0})
    assert F(p0, None, None, None, None, None) == 0
    assert B(p0, None, None, None, None, None, None, None, None, 0, None) == 0
    p0h = _capi.make_problem(**{**BASE, "n": 0, "dtype": _capi.DCN_F16})
    assert _capi.dcn_backward_workspace_size(p0h) == (0, 0)
    assert B(p0h, None, None, None, None, None, None, None, None, 0, None) == 0
    # an invalid problem is reported before the pointers are looked at
    pbad = _capi.make_problem(**{**BASE, "groups": 3})
    assert F(pbad, None, None, None, None, None) == _capi.CODES["DCN_ERR_SHAPE"]


def test_noalloc_backward_checks_before_any_device_call(lib):
    """dcn_backward_noalloc runs dcn_backward's checks on the host; a 16-bit
    image whose fp32 accumulator exceeds the fixed scratch is refused before
    anything is enqueued (the fake pointers are never dereferenced)."""
    m = re.search(r"#define DCN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", HEADER.read_text())
    assert int(m.group(1)) << int(m.group(2)) == _capi.NOALLOC_SCRATCH_BYTES
    NB = _capi.dcn_backward_noalloc
    a = 0x10000
    p = _capi.make_problem(**BASE)
    assert NB(p, a, a, a, a, a, a, None, None) == _capi.CODES["DCN_ERR_NULL"]
    assert NB(p, a, a, a, a, a + 4, a, a, None) == _capi.CODES["DCN_ERR_ALIGN"]
    assert NB(_capi.make_problem(**{**BASE, "groups": 3}), a, a, a, a, a, a, a, None) == _capi.CODES["DCN_ERR_SHAPE"]
    p0 = _capi.make_problem(**{**BASE, "n": 0, "dtype": _capi.DCN_BF16})
    assert NB(p0, None, None, None, None, None, None, None, None) == 0
    # 2048 x 2048 x 16 bf16: a 256 MiB fp32 accumulator per image, above the scratch
    big = _capi.make_problem(**{**BASE, "n": 1, "h": 2048, "w": 2048, "c": 16, "groups": 1,
                                "dtype": _capi.DCN_BF16})
    assert 2048 * 2048 * 16 * 4 > _capi.NOALLOC_SCRATCH_BYTES
    assert NB(big, a, a, a, a, a, a, a, None) == _capi.CODES["DCN_ERR_SCRATCH"]
    assert "scratch" in _capi.dcn_status_string(_capi.CODES["DCN_ERR_SCRATCH"])


def test_fused_forward_checks_before_any_device_call(lib):
    """The fused forwards run dcn_forward's checks plus their own on the host
    (the fake pointers are never dereferenced)."""
    a = 0x10000
    p = _capi.make_problem(**BASE)
    FG, FP = _capi.dcn_forward_generated, _capi.dcn_forward_projected
    for bad_cgd in (0, -8, 12):
        assert FG(p, bad_cgd, a, a, a, None, a, None, a, None) == _capi.CODES["DCN_ERR_SHAPE"], bad_cgd
    assert FG(p, 16, None, a, a, None, a, None, a, None) == _capi.CODES["DCN_ERR_NULL"]
    assert FG(p, 16, a, a, None, None, a, None, a, None) == _capi.CODES["DCN_ERR_NULL"]
    assert FG(p, 16, a, a + 4, a, None, a, None, a, None) == _capi.CODES["DCN_ERR_ALIGN"]
    assert FG(p, 16, a, a, a, a + 2, a, None, a, None) == _capi.CODES["DCN_ERR_ALIGN"]  # fp32 bias
    assert FG(_capi.make_problem(**{**BASE, "groups": 3}), 16, a, a, a, None, a, None, a, None) == \
        _capi.CODES["DCN_ERR_SHAPE"]
    assert FP(p, a, a, a, None, None, a, None) == _capi.CODES["DCN_ERR_NULL"]
    assert FP(p, a, a, a, a + 8, None, a, None) == _capi.CODES["DCN_ERR_ALIGN"]
    p0 = _capi.make_problem(**{**BASE, "n": 0})
    assert FG(p0, 16, None, None, None, None, None, None, None, None) == 0
    assert FP(p0, None, None, None, None, None, None, None) == 0
    # 2560 channels: 16 pixels of fp32 core output (160 KB) leave no room in LDS
    big = _capi.make_problem(**{**BASE, "c": 2560, "groups": 160})
    assert FP(big, a, a, a, a, None, a, None) == _capi.CODES["DCN_ERR_UNSUPPORTED"]


def test_backward_workspace_sizes(lib):
    """The 16-bit backward's fp32 accumulator: one image must stay below 2^31
    bytes, and the workspace covers the largest chunk of images."""
    big = dict(BASE, h=4096, w=4096, c=48, groups=3, dtype=_capi.DCN_BF16, n=1)
    assert _capi.dcn_check(_capi.make_problem(**big))[0] == 0  # the 16-bit tensors fit
    assert _capi.dcn_backward_workspace_size(_capi.make_problem(**big))[0] == _capi.CODES["DCN_ERR_TOO_LARGE"]
    assert _capi.dcn_backward_workspace_size(_capi.make_problem(**dict(big, dtype=_capi.DCN_F32)))[0] == \
        _capi.CODES["DCN_ERR_TOO_LARGE"]  # fp32 input itself too large
    # 2048x1024x64: 512 MiB of fp32 per image, so chunks of 3 images
    chunked = dict(BASE, h=2048, w=1024, c=64, groups=4, dtype=_capi.DCN_F16, n=5)
    assert _capi.dcn_backward_workspace_size(_capi.make_problem(**chunked)) == (0, 3 * 2048 * 1024 * 64 * 4)
    assert _capi.dcn_backward_workspace_size(_capi.make_problem(**dict(chunked, n=2))) == (0, 2 * 2048 * 1024 * 64 * 4)
