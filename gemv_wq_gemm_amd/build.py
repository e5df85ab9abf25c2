"""Builds ``libwq.so`` (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: ``python -m gemv_wq_gemm_amd.build`` (or ``__graft_entry__.build()``).
hipcc cross-compiles for gfx950 without a GPU present.
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
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["wq_api.cpp", "wq_matvec.hip", "wq_matvec_sliced.hip", "wq_matvec_mfma.hip", "wq_matvec_q4k.hip", "wq_gemm.hip",
           "wq_encoder.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed-f32 VALU forms are kept out of the generated code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


# The bench's streaming-read floor: its own library, not part of the layer's ABI.
BENCH_SOURCES = ["bench_read.hip"]
BENCH_LIB = os.path.join(PKG, "libwq_bench.so")


def _link(objs, lib) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link ``gemv_wq_gemm_amd/libwq.so`` (and the bench's
    ``libwq_bench.so``); returns the layer library's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(BENCH_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + BENCH_SOURCES))
    _link(objs[: len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], BENCH_LIB)
    if verbose:
        print(f"built {LIB} and {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
