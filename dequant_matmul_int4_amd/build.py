"""Build libqint4.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m dequant_matmul_int4_amd.build

Every HIP source is compiled for gfx950 only.  Packed-FP32 instruction
selection is disabled (-packed-fp32-ops off); the kernels use scalar and
dot2/MFMA arithmetic instead.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqint4.so")
# measurement aid (the stream-read ceiling bench.py reports), not part of the library
CALIB_LIB = os.path.join(PKG, "libqint4_calib.so")
CALIB_SOURCES = ["calib_read.hip"]
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["api.cpp", "qgemv.hip", "qgemv_mfma.hip", "qgemv_xs.hip", "qgemm.hip", "router.hip", "quant.hip", "moe_prefill.hip",
           "qgemm_stream.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags() -> list:
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I" + INCLUDE, "-I" + CSRC,
    ]


def _compile(src: str) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libqint4.so (and the benchmark's
    calibration library libqint4_calib.so); returns the path of libqint4.so."""
    srcs = SOURCES + CALIB_SOURCES
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIB)
    if verbose:
        print("built", LIB, "and", CALIB_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
