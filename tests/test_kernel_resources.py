"""Register and scratch budget of the hot kernels, read from the gfx950
code the compiler generates (CPU; hipcc cross-compiles).  The kernels are
designed for an occupancy their speed depends on -- the decode attention at
two waves per SIMD, the prompt score GEMM at three, the fused decode index at
a 1024-thread workgroup -- and none may spill to scratch memory.  A change
that silently costs a wave per SIMD or adds spills fails here before it is
timed."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "top_sparse_attention_score_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")

SOURCES = ("qsa_attend_mma.hip", "qsa_index.hip", "qsa_attend.hip", "qsa_append.hip",
           "qsa_window.hip")


def _kernel_info(asm: str) -> dict:
    """{mangled kernel name: {ScratchSize, NumVgprs, Occupancy, ...}} from the
    compiler's per-kernel comment block."""
    info, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1)
            info[cur] = {}
            continue
        m = re.match(r"\s*; (ScratchSize|Occupancy|NumVgprs|TotalNumVgprs|NumAgprs): (\d+)",
                     line)
        if m and cur:
            info[cur][m.group(1)] = int(m.group(2))
    return info


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa")

    def compile_one(src):
        dst = os.path.join(out, src + ".s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "--cuda-device-only", "-S", "-o", dst, os.path.join(CSRC, src)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return _kernel_info(open(dst).read())

    info = {}
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        for part in ex.map(compile_one, SOURCES):
            info.update(part)
    assert len(info) > 100
    return info


def _one(kernels, prefix):
    hits = [v for k, v in kernels.items() if k.startswith(prefix)]
    assert len(hits) == 1, (prefix, len(hits))
    return hits[0]


def test_no_kernel_spills_to_scratch(kernels):
    spilled = sorted(k for k, v in kernels.items() if v.get("ScratchSize", 0) != 0)
    assert not spilled, spilled


@pytest.mark.parametrize("prefix,waves", [
    # decode attention (fp32 q, shared split query) with the merge inside,
    # alone, and with several chunks per wave: two waves per SIMD
    ("_ZN3qsa18k_attend_merge_mmaILi12ELi256ELb0ELb1EE", 2),
    ("_ZN3qsa12k_attend_mmaILi12ELi256ELb0ELb1EE", 2),
    ("_ZN3qsa16k_attend_mch_mmaILi12ELi256ELb0EE", 2),
    # prompt attention (fp16 q)
    ("_ZN3qsa18k_attend_merge_mmaILi12ELi256ELb1ELb0EE", 2),
    # prompt score GEMM keeping candidates: three waves per SIMD
    ("_ZN3qsa13k_idx_collectILi128ELi4EE", 3),
    # fused decode scan + select (+ append): a 1024-thread workgroup needs 4
    ("_ZN3qsa13k_scan_selectILi128ELi8ELb1EE", 4),
    ("_ZN3qsa13k_scan_selectILi128ELi8ELb0EE", 4),
])
def test_hot_kernel_occupancy(kernels, prefix, waves):
    k = _one(kernels, prefix)
    assert k["Occupancy"] >= waves, k
