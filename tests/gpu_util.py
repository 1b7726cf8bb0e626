"""Helpers shared by the GPU tests: run the HIP path through the C ABI on
seeded inputs and compare with the oracle.

Tolerances (fixed by the workload definition for the fp32 attention output):
  out:  max |gpu - oracle| <= 2e-3 and ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2
  ids, n_sel: bit-exact
Partials are checked too, as diagnostics with bounds derived from fp32
arithmetic on these shapes (logits of magnitude <~ 10 summed over <= 256
products): |dm| <= 1e-3 (1 + |m|), |dl| <= 1e-3 l, |d(o/l)| <= 1e-3.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import top_sparse_attention_score_amd as qsa

OUT_ATOL = 2e-3
OUT_REL_L2 = 1e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


# qsa_attend kernel families exercised by the parity tests
ALGOS = {"matrix": qsa.QSA_ATTEND_MATRIX, "vector": qsa.QSA_ATTEND_VECTOR}


def run_gpu(inp: dict, *, P: int | None = None, strides=None, dev=None, ids=None,
            n_sel=None, index=True, algo: str = "matrix", gate=None) -> dict:
    """Runs index_topk -> attend -> merge (gated when a gate array is given)
    on cuda:0 and returns numpy copies."""
    path = qsa.path_for(inp, P=P, strides=strides, algo=ALGOS[algo])
    dev = qsa.to_device(inp) if dev is None else dev
    if index:
        path.index(dev["q_idx"], dev["K_idx"])
    ids_t = path.ids if ids is None else torch.from_numpy(ids).cuda()
    nsel_t = path.n_sel if n_sel is None else torch.from_numpy(n_sel).cuda()
    path.attend(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"], ids=ids_t,
                n_sel=nsel_t)
    path.merge(gate=None if gate is None else torch.from_numpy(np.ascontiguousarray(gate)).cuda())
    torch.cuda.synchronize()
    return dict(ids=path.ids.cpu().numpy(), n_sel=path.n_sel.cpu().numpy(),
                pm=path.pm.cpu().numpy(), pl=path.pl.cpu().numpy(),
                po=path.po.cpu().numpy(), out=path.out.float().cpu().numpy())


def out_errors(gpu: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    diff = gpu.astype(np.float64) - ref
    max_abs = float(np.abs(diff).max())
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel


def assert_out_close(gpu: np.ndarray, ref: np.ndarray, what: str = "out") -> None:
    max_abs, rel = out_errors(gpu, ref)
    assert max_abs <= OUT_ATOL and rel <= OUT_REL_L2, \
        f"{what}: max_abs {max_abs:.3e} (<= {OUT_ATOL}), rel_l2 {rel:.3e} (<= {OUT_REL_L2})"


def assert_ids_equal(gpu_ids, gpu_nsel, ref_ids, ref_nsel) -> None:
    assert np.array_equal(gpu_nsel, ref_nsel), "n_sel differs"
    if not np.array_equal(gpu_ids, ref_ids):
        bad = np.argwhere(gpu_ids != ref_ids)
        raise AssertionError(f"ids differ at {len(bad)} positions, first {bad[:3].tolist()}")


def assert_partials_close(res: dict, pm, pl, po) -> None:
    gm, gl, go = res["pm"].astype(np.float64), res["pl"].astype(np.float64), res["po"]
    empty = np.isneginf(pm)
    assert np.array_equal(np.isneginf(gm), empty), "empty-chunk pattern differs"
    assert np.all(gl[empty] == 0) and np.all(go[empty] == 0)
    full = ~empty
    assert np.all(np.abs(gm[full] - pm[full]) <= 1e-3 * (1 + np.abs(pm[full]))), "m"
    assert np.all(np.abs(gl[full] - pl[full]) <= 1e-3 * pl[full]), "l"
    on = go[full] / gl[full][..., None]
    ro = po[full] / pl[full][..., None]
    assert np.abs(on - ro).max() <= 1e-3, "o/l"
