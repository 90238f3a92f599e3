"""Build step: compile the HIP sources into libdense_gemm_04_amd.so (gfx950 only).

Every translation unit is compiled with hipcc for gfx950 alone, -O3, and with
packed-fp32 instruction selection switched off on the device side. Objects go
to ``_build/`` beside the package and are linked into
``dense_gemm_04_amd/libdense_gemm_04_amd.so``.

Two checking builds of the same sources are linked beside it for the tests
(``build_all``): ``libdense_gemm_04_amd_poison.so`` (DG_LDS_CHECK=1: every
retired LDS stage is filled with NaN) and ``libdense_gemm_04_amd_sync.so``
(DG_LDS_CHECK=2: every global -> LDS copy completes before any wave reads
LDS again). Both must reproduce the normal build bit for bit.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdense_gemm_04_amd.so")
# Checking builds: name -> DG_LDS_CHECK value.
CHECK_BUILDS = {"poison": 1, "sync": 2}


def lib_path(check: str = "") -> str:
    return LIB if not check else os.path.join(PKG, f"libdense_gemm_04_amd_{check}.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, extra, verbose: bool, out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CXXFLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature name; that warning is noise.
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, extra=(), check: str = "") -> str:
    """Compile and link one library: the normal build, or the checking build
    named `check` (a key of CHECK_BUILDS)."""
    out_dir = BUILD_DIR if not check else os.path.join(BUILD_DIR, check)
    flags = list(extra) + ([f"-DDG_LDS_CHECK={CHECK_BUILDS[check]}"] if check else [])
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, flags, verbose, out_dir), srcs))
    lib = lib_path(check)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build_all(verbose: bool = False):
    """The normal library and both checking builds."""
    return [build(verbose)] + [build(verbose, check=c) for c in CHECK_BUILDS]


if __name__ == "__main__":
    print(build_all(verbose="-v" in sys.argv))
