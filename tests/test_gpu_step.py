"""qsa_step -- append -> index -> attend -> gated merge in the fewest launches
the shape allows -- against the same four calls launched one by one,
through the C ABI, on the same seeded inputs: the written cache (codes,
scales, index keys), ids, n_sel and the output must be equal bit for bit.

The cases cover each way the step folds calls: the append inside the
decode scan/select kernel (one token, 128 or more problems, rows of at most
16384 cells), inside the chip-wide one-token scan (fewer problems) or as its
own kernel; the merge inside the attention kernel
(P in {1, 2, 4}; P a multiple of 4 with 512 or more (token, KV head) pairs)
or as its own kernel (other splits, the vector kernel); dense rows; the
draft, long and prompt-chunk index paths; fp16 queries and outputs; no index
keys appended.  Two cases are also checked against the oracle."""
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


ARRAYS = ("q_idx", "K_idx", "q", "Kq", "Ksc", "Vq", "Vsc")

PROMPT_SMALL = dict(T=64, N=4096, di=128, k=256, dense_max=259, Hq=24, Hkv=2, D=256, P=1,
                    q_dtype="f16", out_dtype="f16", heavy_tail=False)
# many tokens through the sampled-bound index (rows of 16384 cells and more)
PROMPT_MID = dict(T=128, N=16384, di=128, k=2048, dense_max=2051, Hq=24, Hkv=2, D=256, P=1,
                  q_dtype="f16", out_dtype="f16", heavy_tail=False)

# (config, batch, P, gate, append index keys, overrides)
CASES = [
    ("decode", 128, 4, True, True, dict(tile=4)),     # append in the scan, merge in attention
    ("decode", 160, 8, True, True, dict(tile=4)),     # append in the scan, separate merge
    ("decode", 128, 4, False, False, dict(tile=4)),   # no gate, no new index key
    ("decode", 2, 4, True, True, {}),                 # append in the chip-wide scan, merge in attention
    ("decode", 3, 4, True, False, {}),                # the same without a new index key
    ("decode", 1, 32, True, True, {}),                # one problem: append in the scan, merge apart
    ("decode", 2, 4, True, True, dict(N=65536)),      # the same over 65536 cells (64 keys a thread)
    ("decode", 3, 16, True, True, {}),                # append in the chip-wide scan, separate merge
    ("decode", 2, 2, True, True, dict(pos0=1500)),    # dense rows
    ("tiny", 5, 4, True, True, {}),
    ("tiny", 130, 1, True, True, dict(tile=5)),       # append in the scan, P = 1
    ("draft", 2, 16, True, True, {}),
    ("long", 1, 64, True, True, dict(pos0=100000)),
    ("prompt_small", 1, 1, True, True, {}),
    ("prompt_mid", 1, 1, True, True, {}),             # sampled-bound index, many tokens
    ("prompt_mid", 2, 1, False, False, {}),           # the same without new index keys
    ("prompt_small", 1, 4, False, True, {}),
    ("decode", 3, 4, True, True, dict(algo=qsa.QSA_ATTEND_VECTOR)),   # vector kernel: merge apart
    ("decode", 128, 8, True, True, dict(tile=4, algo=qsa.QSA_ATTEND_VECTOR)),
]


def _inputs(cfg, seed, B, over):
    over = dict(over)
    tile = over.pop("tile", None)
    over.pop("algo", None)
    c = {"prompt_small": PROMPT_SMALL, "prompt_mid": PROMPT_MID}.get(cfg, cfg)
    if tile is None:
        return make_inputs(c, seed=seed, batch=B, **over)
    inp = make_inputs(c, seed=seed, batch=tile, **over)
    reps = (B + tile - 1) // tile
    for k in ARRAYS:
        inp[k] = np.ascontiguousarray(np.concatenate([inp[k]] * reps)[:B])
    inp["batch"] = B
    return inp


def _new_rows(inp, seed, with_idx, with_gate):
    B, T, Hkv, D, di = inp["batch"], inp["T"], inp["Hkv"], inp["D"], inp["di"]
    g = torch.Generator(device="cuda").manual_seed(seed)
    k_new = torch.randn((B, T, Hkv, D), generator=g, device="cuda")
    v_new = torch.randn((B, T, Hkv, D), generator=g, device="cuda") * 2
    i_new = torch.randn((B, T, di), generator=g, device="cuda") if with_idx else None
    gate = None
    if with_gate:
        gate = torch.randn((B,) + tuple(inp["q"].shape[1:]), generator=g, device="cuda")
        gate = gate.to(torch.float16 if inp["q_dtype"] == "f16" else torch.float32)
    return k_new, v_new, i_new, gate


def _pdesc(inp):
    return qsa.append_desc(batch=inp["batch"], T=inp["T"], n_cells=inp["N"], pos0=inp["pos0"],
                           Hkv=inp["Hkv"], D=inp["D"], d_idx=inp["di"])


def _separate(inp, dev, P, rows, algo=qsa.QSA_ATTEND_AUTO):
    k_new, v_new, i_new, gate = rows
    qsa.qsa_kv_append(_pdesc(inp), k_new, v_new, i_new, dev["Kq"], dev["Ksc"], dev["Vq"],
                      dev["Vsc"], dev["K_idx"])
    path = qsa.path_for(inp, P=P, algo=algo)
    path.run(dict(dev, gate=gate))
    return path


def _step(inp, dev, path, rows, ws=None):
    k_new, v_new, i_new, gate = rows
    need = qsa.qsa_step_workspace(path.idesc, path.adesc)
    assert need > 0
    if ws is None:
        ws = torch.full((need // 4 + 64,), -1, dtype=torch.int32, device="cuda")
    ids = torch.full_like(path.ids, -7)
    n_sel = torch.full_like(path.n_sel, -7)
    out = torch.full_like(path.out, float("nan"))
    qsa.qsa_step(_pdesc(inp), path.idesc, path.adesc, k_new, v_new, i_new, dev["Kq"],
                 dev["Ksc"], dev["Vq"], dev["Vsc"], dev["K_idx"], dev["q_idx"], dev["q"], gate,
                 ids, n_sel, out, ws)
    return ids, n_sel, out, ws


def _same(a, b, what):
    a, b = a.cpu(), b.cpu()
    if a.dtype.is_floating_point:
        it = torch.int16 if a.element_size() == 2 else torch.int32
        a, b = a.view(it), b.view(it)
    assert torch.equal(a, b), f"{what}: {(a != b).sum().item()} elements differ"


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}-P{c[2]}-{i}"
                                             for i, c in enumerate(CASES)])
def test_step_equals_separate_calls(case):
    cfg, B, P, with_gate, with_idx, over = case
    inp = _inputs(cfg, 8100 + B + P, B, over)
    say(f"[step] {cfg} B={B} T={inp['T']} P={P} N={inp['N']} pos0={inp['pos0']} "
        f"gate={with_gate} idx={with_idx}")
    dev_a = qsa.to_device(inp)
    dev_b = {k: v.clone() for k, v in dev_a.items()}
    rows = _new_rows(inp, 41 + B, with_idx, with_gate)
    path = _separate(inp, dev_a, P, rows, over.get("algo", qsa.QSA_ATTEND_AUTO))
    ids, n_sel, out, ws = _step(inp, dev_b, path, rows)
    torch.cuda.synchronize()
    for name in ("Kq", "Ksc", "Vq", "Vsc", "K_idx"):
        _same(dev_a[name], dev_b[name], name)
    _same(path.n_sel, n_sel, "n_sel")
    _same(path.ids, ids, "ids")
    _same(path.out, out, "out")
    # the same step again (the cache already holds the new tokens)
    ids2, n_sel2, out2, _ = _step(inp, dev_b, path, rows, ws=ws)
    torch.cuda.synchronize()
    _same(ids, ids2, "ids (repeat)")
    _same(out, out2, "out (repeat)")


@pytest.mark.parametrize("cfg,B,tile", [("tiny", 3, None), ("decode", 128, 2)])
def test_step_matches_oracle(orc, cfg, B, tile):
    """The step against the oracle: the oracle appends the same rows, then
    runs the path; with 128 problems (append inside the scan kernel) four
    problems are checked."""
    inp = _inputs(cfg, 8300 + B, B, {} if tile is None else dict(tile=tile))
    say(f"[step oracle] {cfg} B={B}")
    P = inp["P"]
    dev = qsa.to_device(inp)
    rows = _new_rows(inp, 88, True, True)
    path = qsa.path_for(inp, P=P)
    ids, n_sel, out, _ = _step(inp, dev, path, rows)
    torch.cuda.synchronize()
    k_new, v_new, i_new, gate = (r.cpu().numpy() for r in rows)
    check = list(range(B)) if B <= 4 else [0, 1, 77, B - 1]
    sub = {k: (inp[k][check] if k in ARRAYS else inp[k]) for k in inp}
    sub["batch"] = len(check)
    rK, rKs, rV, rVs, rI = orc.kv_append(k_new[check], v_new[check], i_new[check], sub["Kq"],
                                         sub["Ksc"], sub["Vq"], sub["Vsc"], sub["K_idx"],
                                         pos0=inp["pos0"])
    assert np.array_equal(dev["Kq"].cpu().numpy()[check], rK)
    assert np.array_equal(dev["Vq"].cpu().numpy()[check], rV)
    assert np.array_equal(dev["Ksc"].cpu().numpy()[check].view(np.uint16), rKs)
    assert np.array_equal(dev["Vsc"].cpu().numpy()[check].view(np.uint16), rVs)
    assert np.array_equal(dev["K_idx"].cpu().numpy()[check].view(np.uint16), rI)
    sub.update(Kq=rK, Ksc=rKs.view(np.float16), Vq=rV, Vsc=rVs.view(np.float16),
               K_idx=rI.view(np.float16))
    ref = orc.run(sub, P=P, scale=1.0 / math.sqrt(inp["D"]))
    assert_ids_equal(ids.cpu().numpy()[check], n_sel.cpu().numpy()[check], ref["ids"],
                     ref["n_sel"])
    want = orc.merge_gated(ref["pm"], ref["pl"], ref["po"], gate[check])
    assert_out_close(out.cpu().numpy()[check], want, f"{cfg} step")


def test_bench_decode_step_configuration(orc):
    """The decode step as the benchmark times it: 512 problems (8 distinct
    seeded caches tiled over the batch), the cell-interleaved cache record
    (1088 bytes per cell), seeded new rows appended, one qsa_step
    call.  Eight problems spread over the batch are checked against the
    oracle (appended codes and scales, ids bit for bit, gated output)."""
    import bench
    B, nd = 512, 8
    base = make_inputs("decode", seed=1234, batch=nd)
    dev = {}
    for key in ARRAYS:
        t = torch.from_numpy(base[key]).cuda()
        dev[key] = t.repeat((B // nd,) + (1,) * (t.dim() - 1)).contiguous()
    inp = dict(base)
    inp["batch"] = B
    N, Hkv, D, P = inp["N"], inp["Hkv"], inp["D"], inp["P"]
    dev, strides = bench.interleave_cache(dev, B, N, Hkv, D)
    say(f"[bench step] decode B={B} record={strides['kq_cell_stride']} B")
    path = qsa.path_for(inp, P=P, strides=strides)
    rows = _new_rows(inp, 4321, True, True)
    k_new, v_new, i_new, gate = rows
    adesc = qsa.append_desc(batch=B, T=inp["T"], n_cells=N, pos0=inp["pos0"], Hkv=Hkv, D=D,
                            d_idx=inp["di"], strides=strides)
    ws = torch.empty(qsa.qsa_step_workspace(path.idesc, path.adesc) // 4 + 64,
                     dtype=torch.int32, device="cuda")
    qsa.qsa_step(adesc, path.idesc, path.adesc, k_new, v_new, i_new, dev["Kq"], dev["Ksc"],
                 dev["Vq"], dev["Vsc"], dev["K_idx"], dev["q_idx"], dev["q"], gate, path.ids,
                 path.n_sel, path.out, ws)
    torch.cuda.synchronize()
    check = [0, 1, 77, 200, 255, 256, 400, 511]
    sub = {k: (base[k][[b % nd for b in check]] if k in ARRAYS else base[k]) for k in base}
    sub["batch"] = len(check)
    kn, vn, inew, g = (r.cpu().numpy()[check] for r in rows)
    rK, rKs, rV, rVs, rI = orc.kv_append(kn, vn, inew, sub["Kq"], sub["Ksc"], sub["Vq"],
                                         sub["Vsc"], sub["K_idx"], pos0=inp["pos0"])
    got = {name: dev[name].cpu().numpy()[check] for name in ("Kq", "Ksc", "Vq", "Vsc", "K_idx")}
    assert np.array_equal(got["Kq"].reshape(rK.shape), rK)
    assert np.array_equal(got["Vq"].reshape(rV.shape), rV)
    assert np.array_equal(got["Ksc"].view(np.uint16).reshape(rKs.shape), rKs)
    assert np.array_equal(got["Vsc"].view(np.uint16).reshape(rVs.shape), rVs)
    assert np.array_equal(got["K_idx"].view(np.uint16), rI)
    sub.update(Kq=rK, Ksc=rKs.view(np.float16), Vq=rV, Vsc=rVs.view(np.float16),
               K_idx=rI.view(np.float16))
    ref = orc.run(sub, P=P, scale=1.0 / math.sqrt(D))
    assert_ids_equal(path.ids.cpu().numpy()[check], path.n_sel.cpu().numpy()[check], ref["ids"],
                     ref["n_sel"])
    want = orc.merge_gated(ref["pm"], ref["pl"], ref["po"], g)
    assert_out_close(path.out.cpu().numpy()[check], want, "bench decode step")
