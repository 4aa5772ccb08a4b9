"""Compile the gfx950 library libpicattn.so in-tree with hipcc.

    python -m position_independent_attention_amd.build

Each translation unit is compiled to an object in _build/ and linked into
position_independent_attention_amd/libpicattn.so (the attention library) or
libpicpeaks.so (machine-peak microbenchmarks for the benchmark).  Flags: -O3, C++17,
--offload-arch=gfx950, and the packed-fp32 target feature switched off for the
device code (hipcc's host pass warns that it does not know the feature);
-fno-honor-nans for the kernel sources; no edge splitting for machine sinking in
the prefill / selection kernels.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpicattn.so")
SOURCES = ["attn_fwd.hip", "attn_decode.hip", "select_fuse.hip", "api.cpp", "block_hash.cpp"]
# machine-peak microbenchmarks (the benchmark's measured denominators), a
# library of their own
PEAKS_LIB = os.path.join(PKG, "libpicpeaks.so")
PEAKS_SOURCES = ["peaks.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Kernel sources only: no NaN canonicalisation before v_max (the kernels use
# +-inf as sentinels but never rely on NaN semantics).  Host code keeps full
# IEEE semantics for argument validation.
KERNEL_FLAGS = ["-fno-honor-nans"]
# The prefill / selection kernels: do not split a rarely taken branch's edge
# to sink work into it.  The tile loop's rare paths (a moved softmax
# reference) would otherwise pull the common path's exp2 out of the region
# where it runs beside the MFMAs.
FILE_FLAGS = {"attn_fwd.hip": ["-mllvm", "-machine-sink-split=0"]}


def flags_for(src: str) -> list:
    """Extra hipcc flags for one source file."""
    return (KERNEL_FLAGS if src.endswith(".hip") else []) + FILE_FLAGS.get(src, [])


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = flags_for(src)
    cmd = [HIPCC] + CFLAGS + extra + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared libraries; returns the path of
    the attention library."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PEAKS_SOURCES], PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
