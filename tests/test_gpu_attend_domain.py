"""Both attention kernels over the value range the cache format and the
library's own quantiser produce: K and V scales from fp16-subnormal (1e-7)
to 8000, queries up to |q| ~ 1e5, scales that change by decades from cell
to cell, and caches written by qsa_kv_append from rows of magnitude 1e-5
and 3e5 (scales up to the thousands).

Tolerance.  The workload's bound (max-abs 2e-3, rel-L2 1e-2) is stated for
values of order one.  fp32 keeps relative precision, so at other
magnitudes the absolute bound is applied to the output in units of its own
RMS: max-abs <= 2e-3 * max(1, rms(ref)); rel-L2 <= 1e-2 as is.  At tiny
magnitudes the rel-L2 bound is the binding one.
"""
import math

import numpy as np
import pytest
import torch

import top_sparse_attention_score_amd as qsa
from datagen import make_inputs
from tests.gpu_util import OUT_ATOL, OUT_REL_L2, out_errors, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _base(seed, q_dtype="f32"):
    return make_inputs("decode", seed=seed, batch=2, N=4096, q_dtype=q_dtype,
                       out_dtype="f32")


def _scales(rng, shape, s):
    return (rng.uniform(0.75, 1.25, size=shape) * s).astype(np.float16)


def _check(orc, inp, algo, tag, dev=None):
    res = run_gpu(inp, algo=algo, dev=dev)
    ref = orc.run(inp, P=inp["P"], scale=1.0 / math.sqrt(inp["D"]))
    assert np.array_equal(res["ids"], ref["ids"]) and np.array_equal(res["n_sel"], ref["n_sel"])
    out = res["out"]
    assert np.all(np.isfinite(out)), f"{tag}: non-finite output"
    rms = float(np.sqrt(np.mean(ref["out"] ** 2)))
    max_abs, rel = out_errors(out, ref["out"])
    atol = OUT_ATOL * max(1.0, rms)
    say(f"[domain] {tag} {algo}: rms {rms:.3e} max_abs {max_abs:.3e} rel_l2 {rel:.3e}")
    assert max_abs <= atol and rel <= OUT_REL_L2, \
        f"{tag} {algo}: max_abs {max_abs:.3e} (<= {atol:.3e}), rel_l2 {rel:.3e}"


SCALES = [1e-7, 1e-4, 1.0, 100.0, 250.0, 1000.0, 8000.0]


@pytest.mark.parametrize("algo", ["matrix", "vector"])
@pytest.mark.parametrize("which", ["V", "K"])
@pytest.mark.parametrize("s", SCALES)
def test_scale_magnitudes(orc, algo, which, s):
    inp = _base(8100 + SCALES.index(s) + (7 if which == "K" else 0))
    rng = np.random.default_rng(8200 + SCALES.index(s))
    key = "Vsc" if which == "V" else "Ksc"
    inp[key] = _scales(rng, inp[key].shape, s)
    _check(orc, inp, algo, f"{which} scales x{s:g}")


@pytest.mark.parametrize("algo", ["matrix", "vector"])
@pytest.mark.parametrize("mag", [1e-4, 1e3, 1e5])
def test_query_magnitudes(orc, algo, mag):
    inp = _base(8300 + int(math.log10(mag)))
    inp["q"] = (inp["q"].astype(np.float64) * mag).astype(np.float32)
    _check(orc, inp, algo, f"|q| x{mag:g}")


@pytest.mark.parametrize("algo", ["matrix", "vector"])
def test_large_query_and_large_scales(orc, algo):
    inp = _base(8400)
    rng = np.random.default_rng(8401)
    inp["q"] = (inp["q"].astype(np.float64) * 3e4).astype(np.float32)
    inp["Vsc"] = _scales(rng, inp["Vsc"].shape, 8000.0)
    inp["Ksc"] = _scales(rng, inp["Ksc"].shape, 1e-4)
    _check(orc, inp, algo, "q x3e4, V x8000, K x1e-4")


@pytest.mark.parametrize("algo", ["matrix", "vector"])
@pytest.mark.parametrize("q_dtype", ["f32", "f16"])
def test_mixed_scales_across_cells(orc, algo, q_dtype):
    """Per-cell V and K scales drawn log-uniformly over ten decades, so the
    largest scale of consecutive 32-cell tiles keeps changing."""
    inp = _base(8500 + (q_dtype == "f16"), q_dtype=q_dtype)
    rng = np.random.default_rng(8501)
    B, N, Hkv, NB = inp["Vsc"].shape
    for key, lo, hi in (("Vsc", -6.0, 4.0), ("Ksc", -3.0, 0.0)):
        cell = 10.0 ** rng.uniform(lo, hi, size=(B, N, 1, 1))
        inp[key] = (cell * rng.uniform(0.75, 1.25, size=(B, N, Hkv, NB))).astype(np.float16)
    _check(orc, inp, algo, f"mixed per-cell scales, q {q_dtype}")


@pytest.mark.parametrize("algo", ["matrix", "vector"])
@pytest.mark.parametrize("mag", [1e-5, 3e5])
def test_appended_cache_magnitudes(orc, algo, mag):
    """The whole cache written by qsa_kv_append from rows of magnitude mag
    (scales ~ mag / 50: fp16-subnormal at 1e-5, thousands at 3e5); the
    oracle's quantiser gives the reference cache."""
    inp = _base(8600 + int(math.log10(mag)))
    B, N, Hkv, D, di = inp["batch"], inp["N"], inp["Hkv"], inp["D"], inp["di"]
    rng = np.random.default_rng(8601)
    k_new = (rng.normal(size=(B, N, Hkv, D)) * mag).astype(np.float32)
    v_new = (rng.normal(size=(B, N, Hkv, D)) * mag).astype(np.float32)
    i_new = inp["K_idx"].astype(np.float32)          # grid values: fp16-exact
    dev = qsa.to_device(inp)
    d = qsa.append_desc(batch=B, T=N, n_cells=N, pos0=0, Hkv=Hkv, D=D, d_idx=di)
    qsa.qsa_kv_append(d, torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda(),
                      torch.from_numpy(i_new).cuda(), dev["Kq"], dev["Ksc"], dev["Vq"],
                      dev["Vsc"], dev["K_idx"])
    torch.cuda.synchronize()
    rK, rKs, rV, rVs, rI = orc.kv_append(k_new, v_new, i_new, inp["Kq"], inp["Ksc"],
                                         inp["Vq"], inp["Vsc"], inp["K_idx"], pos0=0)
    for key, want in (("Kq", rK), ("Vq", rV)):
        assert np.array_equal(dev[key].cpu().numpy(), want), key
    for key, want in (("Ksc", rKs), ("Vsc", rVs), ("K_idx", rI)):
        assert np.array_equal(dev[key].cpu().numpy().view(np.uint16), want), key
    inp.update(Kq=rK, Ksc=rKs.view(np.float16), Vq=rV, Vsc=rVs.view(np.float16),
               K_idx=rI.view(np.float16))
    say(f"[domain] appended x{mag:g}: V scales {rVs.view(np.float16).astype(np.float64).min():.2e}"
        f" .. {rVs.view(np.float16).astype(np.float64).max():.2e}")
    _check(orc, inp, algo, f"appended cache x{mag:g}", dev=dev)
