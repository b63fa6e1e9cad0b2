"""Build libdcn_mi355x.so (the C-ABI library and its gfx950 kernels) in-tree.

Every HIP source is compiled with hipcc for gfx950 only, with packed-fp32
instruction selection disabled, then linked into one shared library next to
this file.  Running this file (or ``__graft_entry__.build()``) always rebuilds.
"""
from __future__ import annotations

import os
import pathlib
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = PKG / "_build"
LIB = PKG / "libdcn_mi355x.so"
SOURCES = ["dcn_api.hip", "dcn_forward.hip", "dcn_fwd_tile.hip", "dcn_fwd_lane.hip", "dcn_fwd_map.hip", "dcn_backward.hip", "dcn_bwd_tile.hip", "dcn_bwd_quad.hip", "dcn_bwd_map.hip", "dcn_fused.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.environ.get("HIPCC", os.path.join(rocm, "bin", "hipcc"))


def compile_flags(extra=()) -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}", *extra]


def build(verbose: bool = False, extra_flags=(), out: pathlib.Path = LIB,
          build_dir: pathlib.Path = BUILD) -> pathlib.Path:
    build_dir.mkdir(parents=True, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = build_dir / (src + ".o")
        cmd = [hipcc(), *compile_flags(extra_flags), "-c", str(CSRC / src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(str(obj))
    failed = []
    for src, pr in procs:
        log = pr.communicate()[0].decode(errors="replace")
        # the host pass does not know the gfx feature flag; that warning is noise
        lines = [ln for ln in log.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or pr.returncode):
            print("\n".join(lines), file=sys.stderr)
        if pr.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = out.with_suffix(".so.tmp")
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
