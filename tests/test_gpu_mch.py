"""GPU tests of the attention kernel's several-chunks-per-wave mapping.

With P a multiple of 4 above 4 and at least 512 (token, KV head) pairs in a
call, one workgroup serves one (token, KV head) and each wave computes
several chunks in turn (the draft batch's shape).  Its partials must equal,
bit for bit, those of the one-chunk-per-wave mapping, which the same
problems get when run in small slices (too few pairs for the other
mapping); qsa_step, which then merges inside the same kernel, must equal
qsa_attend + qsa_merge_gated.  Cases: the draft batch (P = 16), decode
caches at P = 8 and 16, and rows with empty chunks (fewer kept cells than
chunks, and none)."""
import numpy as np
import pytest
import torch

import top_sparse_attention_score_amd as qsa
from datagen import make_inputs, scattered_ids
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

ARRAYS = ("q_idx", "K_idx", "q", "Kq", "Ksc", "Vq", "Vsc")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _tiled(cfg, seed, B, tile, **over):
    inp = make_inputs(cfg, seed=seed, batch=tile, **over)
    reps = (B + tile - 1) // tile
    for k in ARRAYS:
        inp[k] = np.ascontiguousarray(np.concatenate([inp[k]] * reps)[:B])
    inp["batch"] = B
    return inp


def _bits(t):
    return t.contiguous().view(torch.int32).cpu()


def _partials(inp, P, ids, n_sel, dev=None):
    path = qsa.path_for(inp, P=P)
    dev = qsa.to_device(inp) if dev is None else dev
    path.attend(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"], ids=ids, n_sel=n_sel)
    torch.cuda.synchronize()
    return path


def _slice(inp, lo, hi):
    s = {k: (v[lo:hi] if k in ARRAYS else v) for k, v in inp.items()}
    s["batch"] = hi - lo
    return s


@pytest.mark.parametrize("cfg,B,P,tile", [("draft", 32, 16, 4), ("decode", 256, 16, 4),
                                          ("decode", 256, 8, 4)])
def test_several_chunks_per_wave_equal_one_chunk_per_wave(cfg, B, P, tile):
    inp = _tiled(cfg, 470 + P, B, tile)
    T = inp["T"]
    assert B * T * inp["Hkv"] >= 512
    say(f"[mch] {cfg} B={B} T={T} P={P}")
    dev = qsa.to_device(inp)
    path = qsa.path_for(inp, P=P)
    path.index(dev["q_idx"], dev["K_idx"])
    big = _partials(inp, P, path.ids, path.n_sel, dev)
    for lo in (0, 1, B - 1):
        sub = _slice(inp, lo, lo + 1)
        small = _partials(sub, P, path.ids[lo:lo + 1].contiguous(),
                          path.n_sel[lo:lo + 1].contiguous())
        for name in ("pm", "pl", "po"):
            a, b = getattr(big, name)[lo:lo + 1], getattr(small, name)
            assert torch.equal(_bits(a), _bits(b)), f"{name} of problem {lo} differs"


def test_several_chunks_per_wave_with_empty_chunks():
    """Rows of 0, 1, 5, 15, 17 and 100 kept cells at P = 16: chunks past the
    last cell are empty (-inf, 0, 0)."""
    B, P = 256, 16
    inp = _tiled("decode", 480, B, 4, N=4096)
    ids, n_sel = scattered_ids(seed=481, batch=B, T=1, N=4096, cap=inp["cap"],
                               pos0=inp["pos0"], n_max=2048)
    for b, n in zip(range(6), (0, 1, 5, 15, 17, 100)):
        n_sel[b, 0] = n
    ids[n_sel[..., None] <= np.arange(ids.shape[-1])] = -1
    ids_t, nsel_t = torch.from_numpy(ids).cuda(), torch.from_numpy(n_sel).cuda()
    dev = qsa.to_device(inp)
    big = _partials(inp, P, ids_t, nsel_t, dev)
    assert torch.isneginf(big.pm[0]).all() and (big.pl[0] == 0).all()
    for lo in range(7):
        small = _partials(_slice(inp, lo, lo + 1), P, ids_t[lo:lo + 1].contiguous(),
                          nsel_t[lo:lo + 1].contiguous())
        for name in ("pm", "pl", "po"):
            assert torch.equal(_bits(getattr(big, name)[lo:lo + 1]), _bits(getattr(small, name))), \
                f"{name} of problem {lo} (n_sel {n_sel[lo, 0]}) differs"


@pytest.mark.parametrize("cfg,B,P,tile", [("draft", 32, 16, 4), ("decode", 256, 16, 4)])
def test_step_merge_in_the_attention_kernel(cfg, B, P, tile):
    """qsa_step at these shapes merges inside the attention kernel; its
    output equals qsa_attend + qsa_merge_gated bit for bit."""
    inp = _tiled(cfg, 490 + P, B, tile)
    T, Hkv, D, di = inp["T"], inp["Hkv"], inp["D"], inp["di"]
    say(f"[mch step] {cfg} B={B} P={P}")
    dev_a = qsa.to_device(inp)
    dev_b = {k: v.clone() for k, v in dev_a.items()}
    g = torch.Generator(device="cuda").manual_seed(491)
    k_new = torch.randn((B, T, Hkv, D), generator=g, device="cuda")
    v_new = torch.randn((B, T, Hkv, D), generator=g, device="cuda")
    i_new = torch.randn((B, T, di), generator=g, device="cuda")
    gate = torch.randn(tuple(inp["q"].shape), generator=g, device="cuda")
    pdesc = qsa.append_desc(batch=B, T=T, n_cells=inp["N"], pos0=inp["pos0"], Hkv=Hkv, D=D,
                            d_idx=di)
    qsa.qsa_kv_append(pdesc, k_new, v_new, i_new, dev_a["Kq"], dev_a["Ksc"], dev_a["Vq"],
                      dev_a["Vsc"], dev_a["K_idx"])
    path = qsa.path_for(inp, P=P)
    path.run(dict(dev_a, gate=gate))
    ws = torch.empty(qsa.qsa_step_workspace(path.idesc, path.adesc) // 4 + 64,
                     dtype=torch.int32, device="cuda")
    ids, n_sel = torch.full_like(path.ids, -7), torch.full_like(path.n_sel, -7)
    out = torch.full_like(path.out, float("nan"))
    qsa.qsa_step(pdesc, path.idesc, path.adesc, k_new, v_new, i_new, dev_b["Kq"], dev_b["Ksc"],
                 dev_b["Vq"], dev_b["Vsc"], dev_b["K_idx"], dev_b["q_idx"], dev_b["q"], gate,
                 ids, n_sel, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(path.ids.cpu(), ids.cpu()) and torch.equal(path.n_sel.cpu(), n_sel.cpu())
    assert torch.equal(_bits(path.out), _bits(out)), \
        f"{(_bits(path.out) != _bits(out)).sum().item()} output elements differ"
