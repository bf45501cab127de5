"""Build libbwta.so (HIP, gfx950) in-tree with hipcc, and libbwta_probe.so (the
benchmark's measurement kernels, not part of the library).

    python -m binary_ternary_matmul_amd.build          # build if sources changed
    python -m binary_ternary_matmul_amd.build --force  # always rebuild

The library is written for gfx950 only.  Flags:
  -ffp-contract=off       no fused multiply-add: every float op is one IEEE op
  -fhip-fp32-correctly-rounded-divide-sqrt   correctly rounded fp32 division
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed-fp32 VALU ops
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbwta.so")
PROBE_LIB = os.path.join(PKG, "libbwta_probe.so")
PROBE_SOURCES = ["probe.hip"]

SOURCES = ["pack.hip", "gemm_mfma.hip", "gemm_mfma_i8.hip", "gemm_popcount.hip", "gemv_mfma.hip",
           "attention.hip", "bwta_api.cpp"]
HEADERS = ["device_common.hpp", "kernels.hpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbwta.so)")


def common_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
            "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result"]


def _stale(target: str, deps: list[str]) -> bool:
    if not os.path.exists(target):
        return True
    t = os.path.getmtime(target)
    return any(os.path.getmtime(d) > t for d in deps)


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    deps = [os.path.join(CSRC, src), os.path.join(INCLUDE, "bwta.h"),
            os.path.join(INCLUDE, "bwta_probe.h")] + \
        [os.path.join(CSRC, h) for h in HEADERS] + [__file__]
    if _stale(obj, deps):
        cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stderr}")
        os.replace(obj + ".tmp", obj)
    return obj


def build(force: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    if force:
        for f in os.listdir(BUILD):
            if f.endswith(".o"):
                os.remove(os.path.join(BUILD, f))
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, objs[len(SOURCES):])):
        if force or _stale(lib, lib_objs):
            tmp = lib + ".tmp%d" % os.getpid()
            cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
            os.replace(tmp, lib)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    a = ap.parse_args()
    build(force=a.force, verbose=True)
    sys.exit(0)
