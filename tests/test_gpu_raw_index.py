"""GPU parity of the index stage on general fp16 index inputs (no 2^-5 grid).

On grid inputs every fp32 partial sum of a score is exact, so the kernels'
fp32 scores equal the oracle's double scores and ids compare bit for bit.
On general fp16 inputs the products are still exact in fp32 (11 + 11
significant bits), but the sums round, and each kernel variant sums in its
own order (DPP row sums for one token, MFMA for 2 and more).  Any order of
summing n exact products has error at most gamma_n * sum_i |q_i k_i| with
gamma_n = n u / (1 - n u), u = 2^-24.  If the kernel selects exactly on its
own fp32 scores, a cell can be kept by the GPU and not by the oracle (or the
reverse) only when it swapped places with another cell across the k-th
score: then both lie within gamma_n (A_i + A_j) <= 2 gamma_n max_j A_j of the
oracle's k-th score tau, where A_j = sum_i |q_i k_ji|.

The test checks, per token:
  - n_sel equals the oracle's (it does not depend on the scores);
  - the GPU row is a valid selection: ascending distinct visible cells, -1
    after n_sel;
  - every cell in the symmetric difference of the two kept sets has
    |s_j - tau| <= 2 gamma_n max_j A_j (s in double);
  - tokens whose kept set equals the oracle's get the oracle's output
    (max-abs 2e-3, rel-L2 1e-2).
The mismatch counts are printed for the record.
"""
import math

import numpy as np
import pytest
import torch

import top_sparse_attention_score_amd as qsa
from datagen import make_inputs
from tests.gpu_util import assert_out_close, say

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def gamma(n: int) -> float:
    return n * U32 / (1.0 - n * U32)


def _run_tiled(base: dict, batch: int):
    """The path on `batch` problems tiled from the base's distinct ones."""
    nd = base["batch"]
    reps = batch // nd
    dev = {}
    for key in ("q_idx", "K_idx", "q", "Kq", "Ksc", "Vq", "Vsc"):
        t = torch.from_numpy(base[key]).cuda()
        dev[key] = t.repeat((reps,) + (1,) * (t.dim() - 1)).contiguous()
    inp = dict(base)
    inp["batch"] = batch
    path = qsa.path_for(inp)
    path.run(dev)
    torch.cuda.synchronize()
    return path.ids.cpu().numpy(), path.n_sel.cpu().numpy(), path.out.float().cpu().numpy()


def check_bounded(inp, ids, n_sel, out, ref, scores, tag):
    """Applies the bounded-mismatch rule to every problem and token; returns
    (mismatched ids, tokens with a mismatch, tokens)."""
    nd, T, di = inp["q_idx"].shape
    g = 2.0 * gamma(di)
    bad_ids = bad_tok = 0
    for b in range(ids.shape[0]):
        d = b % nd
        qa = np.abs(inp["q_idx"][d].astype(np.float64))
        Ka = np.abs(inp["K_idx"][d].astype(np.float64))
        A = qa @ Ka.T                                     # [T][N]
        assert np.array_equal(n_sel[b], ref["n_sel"][d]), f"{tag} b={b}: n_sel"
        for t in range(T):
            n = int(n_sel[b, t])
            nvis = inp["pos0"] + t + 1
            row = ids[b, t]
            assert np.all(row[n:] == -1), f"{tag} b={b} t={t}: padding"
            kept = row[:n]
            assert n == 0 or (kept[0] >= 0 and kept[-1] < nvis and np.all(np.diff(kept) > 0)), \
                f"{tag} b={b} t={t}: not ascending visible cells"
            want = ref["ids"][d, t, :n]
            if np.array_equal(kept, want):
                assert_out_close(out[b, t], ref["out"][d, t], f"{tag} b={b} t={t}")
                continue
            s = scores[d, t, :nvis]
            tau = s[want].min()
            diff = np.setxor1d(kept, want)
            slack = g * A[t, :nvis].max()
            worst = np.abs(s[diff] - tau).max()
            assert worst <= slack, \
                f"{tag} b={b} t={t}: id off the k-th score by {worst:.3e} > bound {slack:.3e}"
            bad_ids += len(np.setdiff1d(kept, want))
            bad_tok += 1
    return bad_ids, bad_tok, ids.shape[0] * T


CASES = {
    # name: (datagen config, overrides, distinct problems, batch)
    "decode_fused": ("decode", {}, 4, 128),     # fused scan + select (>= 128 tokens)
    "decode": ("decode", {}, 2, 2),             # chip-wide DPP scan + row select
    "draft": ("draft", {}, 1, 1),               # MFMA scan of 8 tokens
    "long": ("long", {}, 1, 1),                 # chip-wide select, planted heavy tail
    "prompt64": ("prompt", dict(T=64), 1, 1),   # MFMA score GEMM, 64-token slice
    "sweep_t4": ("decode", dict(N=32768, T=4, pos0=30000), 1, 1),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_raw_fp16_index_bounded(orc, case):
    cfg, over, nd, batch = CASES[case]
    base = make_inputs(cfg, seed=7100 + len(case), batch=nd, index_grid=False, **over)
    say(f"[raw fp16 index] {case}: B={batch} T={base['T']} N={base['N']}")
    ids, n_sel, out = _run_tiled(base, batch)
    r_ids, r_nsel, scores = orc.index_topk(base["q_idx"], base["K_idx"], k=base["k"],
                                           pos0=base["pos0"], dense_max=base["dense_max"],
                                           cap=base["cap"], want_scores=True)
    pm, pl, po = orc.attend(base["q"], base["Kq"], base["Ksc"], base["Vq"], base["Vsc"],
                            r_ids, r_nsel, P=base["P"], scale=1.0 / math.sqrt(base["D"]))
    ref = dict(ids=r_ids, n_sel=r_nsel, out=orc.merge(pm, pl, po))
    bad_ids, bad_tok, ntok = check_bounded(base, ids, n_sel, out, ref, scores, case)
    say(f"[raw fp16 index] {case}: {bad_ids} ids differ from the oracle in {bad_tok} of "
        f"{ntok} tokens (all within the fp32 summation bound)")
