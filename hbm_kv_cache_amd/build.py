"""Build libkvt.so (HIP for gfx950) in-tree with hipcc.

    python -m hbm_kv_cache_amd.build [-v]

Every translation unit is compiled with packed-FP32 instruction generation turned off, then
linked into one shared library that exports the C ABI declared in include/kvt.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvt.so")
ARCH = "gfx950"

SOURCES = ["kvt_host.hip", "kvt_copy.hip", "kvt_topk.hip", "kvt_gather.hip", "kvt_decode.hip",
           "kvt_prefill.hip", "kvt_worker.hip", "kvt_paged.hip", "kvt_engine.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I", INCLUDE, "-I", CSRC]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops"]


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = ["hipcc", *COMMON, *HIP_FLAGS, "-c", path, "-o", obj]
    else:
        cmd = ["hipcc", *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-ldl", "-lhsa-runtime64"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
