"""The whole path driven by a plain C program (tests/abi_driver.c, built by
build() into tests/bin): it allocates device memory with hipMalloc, calls
qsa_kv_append -> qsa_index_topk -> qsa_attend -> qsa_merge_gated through
include/qsa.h on the default stream with the library's default softmax
scale, and writes the results back.  The oracle checks them: appended codes,
scales and index keys and the kept ids bit for bit, the gated output within
max-abs 2e-3 / rel-L2 1e-2.  The same program also runs qsa_attend_merge on
the same ids and qsa_step from the original inputs and checks, in C, that
they give the four calls' results bit for bit."""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

from datagen import make_inputs
from tests.drivers import ABI_DRIVER
from tests.gpu_util import assert_out_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(ABI_DRIVER):
        pytest.fail(f"{ABI_DRIVER} is missing: run __graft_entry__.build()")


@pytest.mark.parametrize("cfg,batch", [("tiny", 2), ("decode", 2)])
def test_c_driver_whole_path(orc, tmp_path, cfg, batch):
    inp = make_inputs(cfg, seed=8800 + batch, batch=batch)
    B, T, N, Hkv, D, di = inp["batch"], inp["T"], inp["N"], inp["Hkv"], inp["D"], inp["di"]
    pos0 = inp["pos0"]
    rng = np.random.default_rng(8801)
    k_new = rng.normal(size=(B, T, Hkv, D)).astype(np.float32)
    v_new = rng.normal(size=(B, T, Hkv, D)).astype(np.float32)
    i_new = (np.clip(np.rint(rng.normal(size=(B, T, di)) * 32), -128, 128) / 32).astype(np.float32)
    gate = rng.normal(size=inp["q"].shape).astype(np.float32)
    files = dict(q_idx=inp["q_idx"], K_idx=inp["K_idx"], q=inp["q"], Kq=inp["Kq"],
                 Ksc=inp["Ksc"], Vq=inp["Vq"], Vsc=inp["Vsc"], k_new=k_new, v_new=v_new,
                 kidx_new=i_new, gate=gate)
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(tmp_path / name)
    (tmp_path / "shape.txt").write_text(
        f"{B} {T} {N} {di} {inp['k']} {pos0} {inp['dense_max']} {inp['cap']} "
        f"{inp['Hq']} {Hkv} {D} {inp['P']}\n")
    say(f"[c driver] {cfg} B={B}")
    r = subprocess.run([ABI_DRIVER, "run", str(tmp_path)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "gpu run ok" in r.stdout and "step equal" in r.stdout
    assert ("attend_merge equal" in r.stdout) == (inp["P"] in (1, 2, 4))

    rK, rKs, rV, rVs, rI = orc.kv_append(k_new, v_new, i_new, inp["Kq"], inp["Ksc"], inp["Vq"],
                                         inp["Vsc"], inp["K_idx"], pos0=pos0)
    got = {n: np.fromfile(tmp_path / f"{n}.out", dtype=dt).reshape(want.shape)
           for n, dt, want in (("Kq", np.int8, rK), ("Ksc", np.uint16, rKs),
                               ("Vq", np.int8, rV), ("Vsc", np.uint16, rVs))}
    assert np.array_equal(got["Kq"], rK) and np.array_equal(got["Vq"], rV)
    assert np.array_equal(got["Ksc"], rKs) and np.array_equal(got["Vsc"], rVs)
    inp.update(Kq=rK, Ksc=rKs.view(np.float16), Vq=rV, Vsc=rVs.view(np.float16),
               K_idx=rI.view(np.float16))
    ref = orc.run(inp, P=inp["P"], scale=1.0 / math.sqrt(D))
    want = orc.merge_gated(ref["pm"], ref["pl"], ref["po"], gate)
    ids = np.fromfile(tmp_path / "ids.out", dtype=np.int32).reshape(ref["ids"].shape)
    n_sel = np.fromfile(tmp_path / "n_sel.out", dtype=np.int32).reshape(ref["n_sel"].shape)
    out = np.fromfile(tmp_path / "out.out", dtype=np.float32).reshape(want.shape)
    assert np.array_equal(n_sel, ref["n_sel"]) and np.array_equal(ids, ref["ids"])
    assert_out_close(out, want, f"{cfg} via the C driver")
