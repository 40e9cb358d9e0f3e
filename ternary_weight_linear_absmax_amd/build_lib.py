"""Build libbitlinear.so (HIP for gfx950) in-tree with hipcc.

Each translation unit is compiled to an object in parallel, then linked into
``ternary_weight_linear_absmax_amd/libbitlinear.so``.  Packed-FP32 VALU forms
are disabled for device code (``-packed-fp32-ops``); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libbitlinear.so")
# measured machine ceilings for the benchmark, a library of its own
CEILINGS_LIB_PATH = os.path.join(PKG, "libbitlinear_ceilings.so")

SOURCES = ["api.hip", "quant_weights.hip", "quant_act.hip", "gemv.hip", "gemm.hip", "skinny.hip",
           "glue.hip", "backward.hip", "groups.hip", "gemm_wide.hip", "gemv3sum.hip"]
CEILINGS_SOURCES = ["ceilings.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CEILINGS_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in CEILINGS_SOURCES], CEILINGS_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {CEILINGS_LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
