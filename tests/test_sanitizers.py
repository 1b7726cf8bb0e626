"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer, the
discipline of the "round 4 track b: mtp input and hyper-connection fusion"
page ("checks actually run", item 2: no FMA contraction, -fsanitize=
address,undefined, five input patterns: seeded random, signed zeros, mixed
powers of two, alternating signs, tiny inputs).

* The oracle with tests/oracle_patterns.c: every oracle entry point on the
  five patterns, guard words around every output, invariant checks.
* The library's host code (argument validation, size queries, dispatch
  set-up) built with host-only sanitizers, driven by tests/abi_driver.c in
  its host mode (no kernel is launched).
* The same C driver against the regular library build.
"""
import os
import shutil
import subprocess

import pytest

from tests.drivers import ROOT, build_abi_driver

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")
ROCM = "/opt/rocm"
CSRC = os.path.join(ROOT, "top_sparse_attention_score_amd", "csrc")
LIB_SOURCES = ("qsa_api", "qsa_index", "qsa_attend", "qsa_attend_mma", "qsa_append")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{cmd[0]} failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    return r.stdout


def test_oracle_five_patterns_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_patterns"
    _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", *SAN, "-o", str(exe),
          os.path.join(ROOT, "oracle", "qsa_oracle.c"),
          os.path.join(ROOT, "tests", "oracle_patterns.c"), "-lm"])
    out = _run([str(exe)], env=ENV)
    for pat in ("seeded random", "signed zeros", "mixed powers of two", "alternating signs",
                "tiny"):
        assert f"pattern {pat}" in out
    assert "checks passed:" in out


def test_abi_driver_host_checks(tmp_path):
    exe = build_abi_driver(str(tmp_path / "abi_driver"))
    assert "host checks passed" in _run([exe, "host"])


@pytest.mark.skipif(not os.path.exists(f"{ROCM}/bin/hipcc"), reason="needs hipcc")
def test_library_host_code_under_sanitizers(tmp_path):
    hipcc = f"{ROCM}/bin/hipcc"
    clang = f"{ROCM}/llvm/bin/clang"
    objs, procs = [], []
    for src in LIB_SOURCES:
        obj = str(tmp_path / f"{src}.o")
        objs.append(obj)
        procs.append(subprocess.Popen(
            [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-c", os.path.join(CSRC, f"{src}.hip"), "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err
    lib = str(tmp_path / "libqsa.so")
    _run([clang + "++", "-shared", "-fPIC", "-fsanitize=address,undefined", "--hip-link",
          "--offload-arch=gfx950", "-o", lib, *objs, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"])
    exe = str(tmp_path / "abi_driver")
    _run([clang, "-std=c11", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
          f"-I{ROOT}/include", os.path.join(ROOT, "tests", "abi_driver.c"), "-o", exe,
          f"-L{tmp_path}", "-lqsa", f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{ROCM}/lib"])
    assert "host checks passed" in _run([exe, "host"], env=ENV)
