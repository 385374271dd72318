"""Build libpkv.so in-tree: the HIP kernels for gfx950 (hipcc) plus the host block manager
(g++, plain C++); and libpkv_probe.so, the measurement probes bench.py uses (read bandwidth,
matrix-core rate, shader clock).
``python -m paged_kv_cache_306_amd.build`` or ``build()``."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")
PROBE_LIB = os.path.join(PKG, "libpkv_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIP_SOURCES = ["pkv_decode.hip", "pkv_multi_query.hip", "pkv_cache_ops.hip", "pkv_step.hip"]
CXX_SOURCES = ["pkv_alloc.cpp", "pkv_step_check.cpp"]
PROBE_SOURCES = ["pkv_probe.hip"]
# Per-source hipcc flags.  The multi-query kernel keeps its MFMA accumulators in ordinary
# VGPRs (gfx950 MFMAs take C/D there too): with the accumulation-register form the compiler
# copies every accumulator between the two register files on each loop iteration.
EXTRA_HIPCC_FLAGS = {"pkv_multi_query.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                     "pkv_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep hipcc from emitting packed-fp32 VALU ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {cmd[0]} (exit {r.returncode})")
    if verbose and r.stderr.strip():
        sys.stderr.write(r.stderr)


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source, link libpkv.so and libpkv_probe.so next to this file; returns the
    path of libpkv.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([_hipcc(), *HIPCC_FLAGS, *EXTRA_HIPCC_FLAGS.get(src, []), "-I", INCLUDE, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    _link(objs, LIB, verbose)
    probe_objs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([_hipcc(), *HIPCC_FLAGS, *EXTRA_HIPCC_FLAGS.get(src, []), "-I", INCLUDE, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        probe_objs.append(obj)
    _link(probe_objs, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
