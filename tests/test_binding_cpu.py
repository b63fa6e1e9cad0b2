"""The Python binding refuses what the HIP library cannot run, before any
device call, and fails loudly when the library is missing."""
import pathlib
import subprocess
import sys

import pytest
import torch

import deformable_convolution_vision_dcn_amd as dcn
from deformable_convolution_vision_dcn_amd import _capi

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_cpu_tensors_are_refused():
    x = torch.zeros(1, 8, 8, 16)
    off = torch.zeros(1, 8, 8, 1, 9, 2)
    m = torch.zeros(1, 8, 8, 1, 9)
    with pytest.raises(ValueError, match="GPU only"):
        dcn.dcn_forward(x, off, m, groups=1)


def test_dcn_check_reports_shape_and_errors():
    assert dcn.dcn_check((32, 96, 96, 160), groups=10) == (96, 96)
    assert dcn.dcn_check((1, 9, 12, 16), groups=1, stride=2, pad=(0, 1), dilation=(1, 2)) == (4, 5)
    with pytest.raises(dcn.DCNError, match="DCN_ERR_SHAPE"):
        dcn.dcn_check((1, 8, 8, 30), groups=4)
    with pytest.raises(dcn.DCNError, match="DCN_ERR_UNSUPPORTED"):
        dcn.dcn_check((1, 8, 8, 64), groups=2)
    assert dcn.dcn_check((1, 8, 8, 16), groups=1, remove_center=True) == (8, 8)
    with pytest.raises(dcn.DCNError, match="DCN_ERR_ARG"):
        dcn.dcn_check((1, 8, 8, 16), groups=1, kernel=(3, 4), pad=(1, 2), remove_center=True)


def test_missing_library_fails_loudly(tmp_path):
    code = ("import deformable_convolution_vision_dcn_amd as d\n"
            "try:\n    d.dcn_abi_version()\nexcept d.LibraryMissing as e:\n    print('LOUD', e)\n")
    env = {"DCN_MI355X_LIB": str(tmp_path / "nope.so"), "PATH": "/usr/bin:/bin"}
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True)
    assert "LOUD" in r.stdout and "no fallback" in r.stdout, r.stdout + r.stderr


def test_package_does_not_import_the_oracle():
    code = ("import sys, deformable_convolution_vision_dcn_amd.ops, "
            "deformable_convolution_vision_dcn_amd._capi\n"
            "print('oracle' in sys.modules)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert r.stdout.strip() == "False", r.stdout + r.stderr


def test_overlap_detection():
    """Outputs that share bytes with another tensor are refused before any
    call (the check runs on byte ranges, so CPU tensors exercise it)."""
    from deformable_convolution_vision_dcn_amd import ops

    base = torch.zeros(1024)
    a, b, c = base[:512], base[256:768], base[512:]
    assert ops._overlaps(a, b) and ops._overlaps(b, c)
    assert not ops._overlaps(a, c)
    assert not ops._overlaps(a, torch.zeros(0))
    with pytest.raises(ValueError, match="overlaps"):
        ops._no_alias([("out", b)], [("input", a)])
    ops._no_alias([("out", c)], [("input", a)])


def test_graft_build_entry_checks_the_built_library(monkeypatch):
    """build()'s steps after compiling (import, ABI version check) run against
    the library already built here; the compile steps are stubbed out."""
    import __graft_entry__ as g
    import oracle.build
    from deformable_convolution_vision_dcn_amd import build as libbuild
    monkeypatch.setattr(libbuild, "build", lambda **kw: None)
    monkeypatch.setattr(oracle.build, "build", lambda **kw: None)
    g.build()
