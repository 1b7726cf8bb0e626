"""Builds of the C test drivers (test infrastructure).

abi_driver   a plain C caller of libqsa.so (tests/abi_driver.c), linked
             against the in-tree library; build() puts it in tests/bin so the
             GPU tests can run it without compiling anything.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BIN = os.path.join(HERE, "bin")
ABI_DRIVER = os.path.join(BIN, "abi_driver")
ROCM = "/opt/rocm"


def build_abi_driver(out: str = ABI_DRIVER, lib_dir: str | None = None) -> str:
    lib_dir = lib_dir or os.path.join(ROOT, "top_sparse_attention_score_amd")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-std=c11", "-O2", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{ROOT}/include", os.path.join(HERE, "abi_driver.c"), "-o", out,
           f"-L{lib_dir}", "-lqsa", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{ROCM}/lib"]
    subprocess.run(cmd, check=True)
    return out
