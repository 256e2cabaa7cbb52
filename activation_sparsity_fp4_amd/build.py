"""Build the SharQ HIP library (libsharq.so) in-tree for gfx950 with hipcc.

Usage: python -m activation_sparsity_fp4_amd.build   (or build() from Python)
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsharq.so")
SOURCES = ["prepare.hip", "gemm.hip", "glue.hip", "compact.hip", "nvfp4.hip", "layout.hip", "scratchfree.hip", "sharq_api.hip"]
CALIB_SOURCE = "calib.hip"
CALIB_LIB = os.path.join(PKG, "libsharq_calib.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU forms.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-fvisibility=hidden",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libsharq.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    # the benchmark's MFMA-rate calibration kernel, a shared object of its own
    obj = _compile(CALIB_SOURCE)
    tmp = CALIB_LIB + ".tmp"
    res = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
