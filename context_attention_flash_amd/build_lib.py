"""Builds libringattn.so (HIP kernels for gfx950 + the host C ABI) in-tree,
and libraprobe.so (the MFMA-only peak probe that bench.py measures with).

Usage: python -m context_attention_flash_amd.build_lib [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libringattn.so")
PROBE_LIB = os.path.join(PKG, "libraprobe.so")
PROBE_SOURCES = ["peak_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.cpp", "planner.cpp", "fwd_bf16.hip", "fwd_f32.hip", "elementwise.hip",
           "bwd_bf16.hip", "noalloc.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
          "--offload-arch=gfx950",
          # keep the compiler away from packed fp32 instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
# Kernel sources only: no value in the kernels is ever NaN, and without this
# every fmaxf first quiets its operands (one extra instruction per value).  The
# host sources keep IEEE semantics (argument checks test for NaN).
KERNEL_ONLY = ["-fno-honor-nans"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = KERNEL_ONLY if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, flush=True)
    return obj


def _link(objs, out: str) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{res.stdout}\n{res.stderr}")
    # every kernel launched from host code must have its launch stub in the
    # library (a stub the host pass failed to emit only shows up at load time)
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "__device_stub__" in ln]
    if nm.returncode != 0 or missing:
        raise RuntimeError(f"library check failed: {nm.stderr.strip()} undefined kernel stubs {missing}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    return _link([objs[s] for s in SOURCES], LIB)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
