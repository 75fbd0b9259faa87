"""Ahead-of-time build of the row-reduction library for gfx950.

Compiles each translation unit with hipcc (in parallel) and links
``libnt.so`` next to this file.  Usage: ``python -m row_wise_reductions_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libnt.so")
CALIB_PATH = os.path.join(HERE, "libntcal.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# Packed fp32 ops are disabled on purpose: the kernels are written as scalar
# fp32/fp64 code and must not be turned into v_pk_* arithmetic.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]

UNITS = [
    ("kernels_f32.o", "kernels_inst.hip", ["-DNTK_DT=0"]),
    ("kernels_f16.o", "kernels_inst.hip", ["-DNTK_DT=1"]),
    ("kernels_bf16.o", "kernels_inst.hip", ["-DNTK_DT=2"]),
    ("attention.o", "attention.hip", []),
    ("nt_api.o", "nt_api.cpp", ["-x", "hip"]),
]


def _compile(unit, extra_flags=(), build_dir=BUILD_DIR):
    obj, src, defs = unit
    out = os.path.join(build_dir, obj)
    cmd = [HIPCC, *COMMON, *defs, *extra_flags, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} {defs}:\n{r.stderr}")
    return out


def build(verbose: bool = True, extra_flags=(), out: str = LIB_PATH, build_dir: str = BUILD_DIR) -> str:
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(UNITS), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda u: _compile(u, extra_flags, build_dir), UNITS))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    if out == LIB_PATH:
        build_calibration(verbose)
    return out


def build_calibration(verbose: bool = True) -> str:
    """The reference copy kernel (libntcal.so), used by bench.py --calibrate."""
    tmp = CALIB_PATH + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", os.path.join(CSRC, "calib_copy.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for calib_copy.hip:\n{r.stderr}")
    os.replace(tmp, CALIB_PATH)
    if verbose:
        print(f"built {CALIB_PATH}")
    return CALIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
