"""Builds libqgemm.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m weight_quantized_gemm_amd.build_lib  (or build() from Python).
Always recompiles; objects go to _build/ at the repository root.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libqgemm.so")
# measured-peak probes for the bench (no GEMM code; never linked into libqgemm.so)
PROBE_OUT = os.path.join(PKG, "libqgemm_probe.so")
PROBE_SOURCES = ["probe.hip"]
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.hip", "gemv.hip", "gemm_int4.hip", "gemm_int8.hip", "w4a8.hip", "gemm_f32.hip", "splitk.hip",
           "quantize.hip", "host_pack.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}"]
# Device code: gfx950 only, no packed-fp32 instructions.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-mcode-object-version=5",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Host-only code (quantiser, packer): no contraction into FMA.
CPP_FLAGS = ["-ffp-contract=off"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *HIP_FLAGS, "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *CPP_FLAGS, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, (os.cpu_count() or 2)), 8)
    with ThreadPoolExecutor(jobs) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], OUT, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_OUT, verbose)
    return OUT


if __name__ == "__main__":
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        sys.exit(f"hipcc not found at {HIPCC}")
    build(verbose=True)
