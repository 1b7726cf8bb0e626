"""qsa_decode_window -- the decode step (append -> index -> attend -> gated
merge) in one cooperative launch -- against the same four calls launched
one by one, through the C ABI, on the same seeded inputs: the written cache
(codes, scales, index keys), ids, n_sel and the output must be equal bit for
bit, and the window's status word must read 0.  Calls run back to back with
changing shapes (the grid barrier's words must come back to their start
state after every call); one case is also checked against the oracle.
With 128 or more problems of at most 16384 cells the separate index call
scores on the matrix cores, in another fp32 summation order than the
window's scan, so those cases use fp16 index inputs on the 2^-5 grid, where
every order gives the exact score."""
import math

import numpy as np
import pytest
import torch

import top_sparse_attention_score_amd as qsa
from datagen import make_inputs
from tests.gpu_util import assert_ids_equal, assert_out_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


# (config, batch, P, gate, new index key, fp16 grid index inputs, overrides)
CASES = [
    ("decode", 1, 32, True, True, True, {}),
    ("decode", 3, 16, False, True, False, {}),
    ("decode", 2, 4, True, False, True, {}),
    ("tiny", 5, 4, True, True, True, {}),
    ("tiny", 2, 8, False, True, False, dict(pos0=100)),       # dense rows (101 <= k)
    ("decode", 2, 32, True, True, True, dict(pos0=1500)),     # dense rows (<= 2051)
    ("decode", 1, 64, True, True, False, dict(N=20000, pos0=16383)),  # longest row
    ("long", 1, 64, True, True, True, dict(pos0=9000)),
    ("decode", 2, 32, True, True, False, dict(pos0=4000)),
    ("decode", 160, 32, True, True, True, dict(tile=4)),       # many problems
    ("tiny", 200, 4, True, True, True, dict(tile=8)),
]

ARRAYS = ("q_idx", "K_idx", "q", "Kq", "Ksc", "Vq", "Vsc")


def _inputs(cfg, seed, B, grid, over):
    """Seeded inputs; with `tile`, B problems repeat that many distinct ones
    (keeps generation fast at large B)."""
    over = dict(over)
    tile = over.pop("tile", None)
    if tile is None:
        return make_inputs(cfg, seed=seed, batch=B, index_grid=grid, **over)
    inp = make_inputs(cfg, seed=seed, batch=tile, index_grid=grid, **over)
    reps = (B + tile - 1) // tile
    for k in ARRAYS:
        inp[k] = np.ascontiguousarray(np.concatenate([inp[k]] * reps)[:B])
    inp["batch"] = B
    return inp


def _new_rows(inp, seed, with_idx, with_gate):
    B, Hkv, D, di, Hq = inp["batch"], inp["Hkv"], inp["D"], inp["di"], inp["Hq"]
    g = torch.Generator(device="cuda").manual_seed(seed)
    k_new = torch.randn((B, 1, Hkv, D), generator=g, device="cuda")
    v_new = torch.randn((B, 1, Hkv, D), generator=g, device="cuda") * 2
    i_new = torch.randn((B, 1, di), generator=g, device="cuda") if with_idx else None
    gate = torch.randn((B, 1, Hq, D), generator=g, device="cuda") if with_gate else None
    return k_new, v_new, i_new, gate


def _pdesc(inp):
    return qsa.append_desc(batch=inp["batch"], T=1, n_cells=inp["N"], pos0=inp["pos0"],
                           Hkv=inp["Hkv"], D=inp["D"], d_idx=inp["di"])


def _multi(inp, dev, P, rows):
    k_new, v_new, i_new, gate = rows
    qsa.qsa_kv_append(_pdesc(inp), k_new, v_new, i_new, dev["Kq"], dev["Ksc"], dev["Vq"],
                      dev["Vsc"], dev["K_idx"])
    path = qsa.path_for(inp, P=P)
    path.run(dict(dev, gate=gate))
    return path


def _window(inp, dev, path, rows, ws=None):
    k_new, v_new, i_new, gate = rows
    B, cap, Hq, D = inp["batch"], inp["cap"], inp["Hq"], inp["D"]
    need = qsa.qsa_decode_window_workspace(path.idesc, path.adesc)
    assert need > 0
    if ws is None:
        ws = torch.full((need // 4 + 64,), -1, dtype=torch.int32, device="cuda")
    ids = torch.full((B, 1, cap), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((B, 1), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, 1, Hq, D), float("nan"), device="cuda")
    qsa.qsa_decode_window(_pdesc(inp), path.idesc, path.adesc, k_new, v_new, i_new, dev["Kq"],
                          dev["Ksc"], dev["Vq"], dev["Vsc"], dev["K_idx"], dev["q_idx"],
                          dev["q"], gate, ids, n_sel, out, ws)
    return ids, n_sel, out, ws


def _same(a, b, what):
    a, b = a.cpu(), b.cpu()
    if a.dtype.is_floating_point:
        it = torch.int16 if a.element_size() == 2 else torch.int32
        a, b = a.view(it), b.view(it)
    assert torch.equal(a, b), f"{what}: {(a != b).sum().item()} elements differ"


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}-P{c[2]}-{i}"
                                             for i, c in enumerate(CASES)])
def test_window_equals_separate_calls(case):
    cfg, B, P, with_gate, with_idx, grid, over = case
    inp = _inputs(cfg, 7100 + B + P, B, grid, over)
    say(f"[window] {cfg} B={B} P={P} N={inp['N']} pos0={inp['pos0']} gate={with_gate} "
        f"idx={with_idx} grid={grid}")
    dev_a = qsa.to_device(inp)
    dev_b = {k: v.clone() for k, v in dev_a.items()}
    rows = _new_rows(inp, 31 + B, with_idx, with_gate)
    path = _multi(inp, dev_a, P, rows)
    ids, n_sel, out, ws = _window(inp, dev_b, path, rows)
    torch.cuda.synchronize()
    assert ws[0].item() == 0, "a grid barrier wait gave up"
    for name in ("Kq", "Ksc", "Vq", "Vsc", "K_idx"):
        _same(dev_a[name], dev_b[name], name)
    _same(path.n_sel, n_sel, "n_sel")
    _same(path.ids, ids, "ids")
    _same(path.out, out, "out")
    # the same step again reuses the workspace and the barrier words
    ids2, n_sel2, out2, _ = _window(inp, dev_b, path, rows, ws=ws)
    torch.cuda.synchronize()
    assert ws[0].item() == 0
    _same(ids, ids2, "ids (repeat)")
    _same(out, out2, "out (repeat)")


@pytest.mark.parametrize("cfg,B", [("tiny", 3), ("decode", 2)])
def test_window_matches_oracle(orc, cfg, B):
    inp = make_inputs(cfg, seed=7300 + B, batch=B)
    say(f"[window oracle] {cfg} B={B}")
    P = inp["P"] if cfg == "tiny" else 32
    dev = qsa.to_device(inp)
    rows = _new_rows(inp, 77, True, True)
    path = qsa.path_for(inp, P=P)
    ids, n_sel, out, ws = _window(inp, dev, path, rows)
    torch.cuda.synchronize()
    assert ws[0].item() == 0
    k_new, v_new, i_new, gate = (r.cpu().numpy() for r in rows)
    rK, rKs, rV, rVs, rI = orc.kv_append(k_new, v_new, i_new, inp["Kq"], inp["Ksc"], inp["Vq"],
                                         inp["Vsc"], inp["K_idx"], pos0=inp["pos0"])
    assert np.array_equal(dev["Kq"].cpu().numpy(), rK)
    assert np.array_equal(dev["Vq"].cpu().numpy(), rV)
    assert np.array_equal(dev["Ksc"].cpu().numpy().view(np.uint16), rKs)
    assert np.array_equal(dev["Vsc"].cpu().numpy().view(np.uint16), rVs)
    assert np.array_equal(dev["K_idx"].cpu().numpy().view(np.uint16), rI)
    inp.update(Kq=rK, Ksc=rKs.view(np.float16), Vq=rV, Vsc=rVs.view(np.float16),
               K_idx=rI.view(np.float16))
    ref = orc.run(inp, P=P, scale=1.0 / math.sqrt(inp["D"]))
    assert_ids_equal(ids.cpu().numpy(), n_sel.cpu().numpy(), ref["ids"], ref["n_sel"])
    want = orc.merge_gated(ref["pm"], ref["pl"], ref["po"], gate)
    assert_out_close(out.cpu().numpy(), want, f"{cfg} window")
