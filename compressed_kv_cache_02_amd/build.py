"""Build libcsa2.so in-tree with hipcc for gfx950.

Usage: python -m compressed_kv_cache_02_amd.build   (or call build()).
Every HIP source is compiled with packed-FP32 instructions disabled; the C-ABI
layer is compiled as HIP host code. The library lands next to this file.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcsa2.so")

ARCH = "gfx950"
HIP_SOURCES = ["quantize_kv.hip", "write_path.hip", "index_score.hip", "select.hip",
               "sparse_attn.hip"]
HOST_SOURCES = ["csa2_api.cpp"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", CSRC, "-I", INCLUDE, "-Wall",
          "-Wno-unused-function"]
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n%s\n%s" % (" ".join(cmd), r.stdout))
    return r.stdout


def build(verbose=False):
    """Compile every source and link libcsa2.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, s + ".o")
        jobs.append((obj, [hipcc, "-c", "-x", "hip", os.path.join(CSRC, s), "-o", obj] + COMMON + DEVICE_FLAGS))
    for s in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, s + ".o")
        jobs.append((obj, [hipcc, "-c", "-x", "hip", os.path.join(CSRC, s), "-o", obj] + COMMON + DEVICE_FLAGS))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                sys.stdout.write(o)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-o", tmp] + [j[0] for j in jobs] + ["--offload-arch=" + ARCH])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
