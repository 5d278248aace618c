"""Build libbase_layer.so (gfx950) in-tree with hipcc, and its checking
variant libbase_layer_checks.so (compiled with BASE_CHECKS: the auction's
kernels verify its invariants on the device and report a failure as
BASE_ERR_INVARIANT).

    python -m balanced_token_expert_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libbase_layer.so")
LIB_CHECKS = os.path.join(HERE, "libbase_layer_checks.so")
SOURCES = ["gemm.hip", "route.hip", "auction.hip", "layernorm.hip", "grad.hip", "api.cpp"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # keep the compiler from forming packed fp32 math (v_pk_*_f32)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(src: str, checks: bool = False) -> str:
    out = os.path.join(BUILD, "checks") if checks else BUILD
    os.makedirs(out, exist_ok=True)
    obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
    extra = ["-DBASE_CHECKS"] if checks else []
    cmd = [_hipcc(), *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, checks: bool = True) -> str:
    """Build the library (and, unless checks=False, its checking variant)."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + ([(src, True) for src in SOURCES] if checks else [])
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    if verbose:
        print(f"built {LIB}")
    if checks:
        _link(objs[n:], LIB_CHECKS)
        if verbose:
            print(f"built {LIB_CHECKS}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
