"""Ahead-of-time build of libqsa.so for gfx950 with hipcc.

Each HIP source is compiled to an object in parallel, then linked into
``top_sparse_attention_score_amd/libqsa.so`` (in-tree, so it travels with the
source tree).  Packed-fp32 instruction selection is disabled for all device
code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqsa.so")
# Bandwidth probe library (measurement only; see csrc/hbm_probe.hip).
PROBE_SRC = "hbm_probe.hip"
PROBE_LIB = os.path.join(PKG, "libhbm_probe.so")

SOURCES = ("qsa_api.hip", "qsa_index.hip", "qsa_attend.hip", "qsa_attend_mma.hip", "qsa_append.hip",
           "qsa_window.hip")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    """Compile every source and link libqsa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe()
    return LIB


def build_probe() -> str:
    """Compile and link libhbm_probe.so (the HBM read-rate probe)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = _compile(PROBE_SRC)
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build())
