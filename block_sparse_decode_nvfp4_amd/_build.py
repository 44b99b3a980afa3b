"""Build libm3s.so (HIP kernels for gfx950 + the C-ABI host layer) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libm3s.so")

HIP_SOURCES = ["store.hip", "producer.hip", "rows.hip", "index_topk.hip", "attend.hip", "probe.hip", "scratch.hip"]
HOST_SOURCES = ["api.cpp"]
HEADERS = ["fp4.hpp", "launch.hpp", "quant.hpp", "rows_body.hpp", "store_body.hpp"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
# Packed fp32 VALU forms are kept out of the generated code (they are not used
# by the kernels; the flag is a device target feature, the host pass ignores it).
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if p.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libm3s.so. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append([_hipcc(), *DEVICE, *COMMON, "-c", os.path.join(CSRC, s), "-o", o])
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append([_hipcc(), "-x", "c++", *COMMON, "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, s), "-o", o])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o:
                print(o, file=sys.stderr)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
