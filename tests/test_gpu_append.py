"""GPU parity of qsa_kv_append: the quantised codes, fp16 scales and fp16
index keys written by the HIP kernel equal the double oracle's bit for bit
(integer and bit-pattern work), untouched cells stay untouched, and a cache
filled by appends feeds the whole path to the oracle's result."""
import math

import numpy as np
import pytest
import torch

import top_sparse_attention_score_amd as qsa
from datagen import make_inputs
from tests.gpu_util import assert_ids_equal, assert_out_close, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _rand_cache(rng, B, N, Hkv, D, di):
    Kq = rng.integers(-127, 128, size=(B, N, Hkv, D)).astype(np.int8)
    Vq = rng.integers(-127, 128, size=(B, N, Hkv, D)).astype(np.int8)
    Ksc = rng.integers(0, 0x7000, size=(B, N, Hkv, D // 32)).astype(np.uint16)
    Vsc = rng.integers(0, 0x7000, size=(B, N, Hkv, D // 32)).astype(np.uint16)
    Kix = rng.integers(0, 0x7000, size=(B, N, di)).astype(np.uint16)
    return Kq, Ksc, Vq, Vsc, Kix


def _gpu_append(k_new, v_new, i_new, Kq, Ksc, Vq, Vsc, Kix, pos0, strides=None):
    B, T, Hkv, D = k_new.shape
    N, di = Kq.shape[1], Kix.shape[-1]
    def _t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
    dev = [_t(a) for a in (Kq, Ksc, Vq, Vsc, Kix)]
    kn = torch.from_numpy(k_new).cuda()
    vn = torch.from_numpy(v_new).cuda()
    inn = torch.from_numpy(i_new).cuda() if i_new is not None else None
    d = qsa.append_desc(batch=B, T=T, n_cells=N, pos0=pos0, Hkv=Hkv, D=D, d_idx=di,
                        strides=strides)
    qsa.qsa_kv_append(d, kn, vn, inn, dev[0], dev[1], dev[2], dev[3], dev[4])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in dev]


@pytest.mark.parametrize("mag", [3e-9, 2e-7, 1e-3, 1.0, 40.0, 3e5])
@pytest.mark.parametrize("D", [64, 256])
def test_append_matches_oracle_bitwise(orc, mag, D):
    rng = np.random.default_rng(int(mag * 1e9) % 1000 + D)
    B, N, T, Hkv, di, pos0 = 3, 40, 5, 2, 128, 17
    say(f"[append] D={D} magnitude={mag}")
    cache = _rand_cache(rng, B, N, Hkv, D, di)
    k_new = (rng.normal(size=(B, T, Hkv, D)) * mag).astype(np.float32)
    v_new = (rng.standard_t(3, size=(B, T, Hkv, D)) * mag).astype(np.float32)
    k_new[0, 0, 0, :32] = 0.0                                  # an all-zero block
    v_new[1, 2, 1, 5] = mag * 1e4                              # one dominant element
    i_new = (rng.normal(size=(B, T, di)) * max(mag, 1e-3)).astype(np.float32)
    got = _gpu_append(k_new, v_new, i_new, *cache, pos0=pos0)
    ref = orc.kv_append(k_new, v_new, i_new, *cache, pos0=pos0)
    for name, g, r in zip(("Kq", "Ksc", "Vq", "Vsc", "K_idx"), got, ref):
        assert np.array_equal(g.view(np.uint8), np.asarray(r).view(np.uint8)), name


def test_append_constructed_ties(orc):
    """Quotients x / s that are exact half-integers go to the even code."""
    B, N, T, Hkv, D, di = 1, 4, 1, 1, 64, 4
    rng = np.random.default_rng(5)
    cache = _rand_cache(rng, B, N, Hkv, D, di)
    k_new = np.zeros((B, T, Hkv, D), np.float32)
    for blk, s in enumerate((0.5, 3.0)):
        x = k_new[0, 0, 0, 32 * blk: 32 * blk + 32]
        x[0] = 127 * s
        for i, hv in enumerate((0.5, 1.5, 2.5, 3.5, 10.5, 125.5)):
            x[1 + i] = hv * s
            x[7 + i] = -hv * s
    v_new = -k_new
    i_new = np.array([[[1e-8, 65519.0, -0.1, 3.14159]]], np.float32)
    got = _gpu_append(k_new, v_new, i_new, *cache, pos0=2)
    ref = orc.kv_append(k_new, v_new, i_new, *cache, pos0=2)
    for name, g, r in zip(("Kq", "Ksc", "Vq", "Vsc", "K_idx"), got, ref):
        assert np.array_equal(g.view(np.uint8), np.asarray(r).view(np.uint8)), name
    assert list(got[0][0, 2, 0, 1:7]) == [0, 2, 2, 4, 10, 126]


def test_append_interleaved_layout_and_no_index(orc):
    """Codes and scales of a cell interleaved in one record via the strides;
    with no index keys given, K_idx is not touched."""
    B, N, T, Hkv, D, di, pos0 = 2, 16, 3, 2, 256, 128, 7
    rec = Hkv * D + Hkv * (D // 32) * 2
    rng = np.random.default_rng(9)
    k_new = rng.normal(size=(B, T, Hkv, D)).astype(np.float32)
    v_new = rng.normal(size=(B, T, Hkv, D)).astype(np.float32)
    buf_k = torch.zeros((B, N, rec), dtype=torch.uint8, device="cuda")
    buf_v = torch.zeros((B, N, rec), dtype=torch.uint8, device="cuda")
    Kix = torch.full((B, N, di), 7, dtype=torch.int16, device="cuda")
    strides = dict(kq_cell_stride=rec, ksc_cell_stride=rec, vq_cell_stride=rec,
                   vsc_cell_stride=rec, kq_batch_stride=N * rec, ksc_batch_stride=N * rec,
                   vq_batch_stride=N * rec, vsc_batch_stride=N * rec)
    d = qsa.append_desc(batch=B, T=T, n_cells=N, pos0=pos0, Hkv=Hkv, D=D, d_idx=di,
                        strides=strides)
    qsa.qsa_kv_append(d, torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda(), None,
                      buf_k, buf_k[:, :, Hkv * D:], buf_v, buf_v[:, :, Hkv * D:], Kix)
    torch.cuda.synchronize()
    assert (Kix == 7).all()
    zero = np.zeros((B, N, Hkv, D), np.int8)
    zs = np.zeros((B, N, Hkv, D // 32), np.uint16)
    rK, rKs, rV, rVs, _ = orc.kv_append(k_new, v_new, np.zeros((B, T, di), np.float32),
                                        zero, zs, zero, zs, np.zeros((B, N, di), np.uint16),
                                        pos0=pos0)
    bk, bv = buf_k.cpu().numpy(), buf_v.cpu().numpy()
    for buf, codes, scales in ((bk, rK, rKs), (bv, rV, rVs)):
        assert np.array_equal(buf[:, :, :Hkv * D].view(np.int8).reshape(B, N, Hkv, D), codes)
        assert np.array_equal(buf[:, :, Hkv * D:].view(np.uint16).reshape(B, N, Hkv, D // 32),
                              scales)


def test_appended_cache_feeds_the_path(orc):
    """Fill a cache token by token with qsa_kv_append from float K / V / index
    rows, then run index_topk -> attend -> merge on it: ids bit-exact and the
    output within tolerance of the oracle on the oracle-appended cache."""
    B, N, Hkv, D, di = 2, 2304, 2, 256, 128
    cfg = dict(T=1, N=N, di=di, k=256, dense_max=259, Hq=24, Hkv=Hkv, D=D, P=4,
               q_dtype="f32", out_dtype="f32", heavy_tail=False)
    inp = make_inputs(cfg, seed=91, batch=B)
    rng = np.random.default_rng(92)
    k_all = rng.normal(size=(B, N, Hkv, D)).astype(np.float32)
    v_all = rng.normal(size=(B, N, Hkv, D)).astype(np.float32)
    # index keys on the 2^-5 grid so the scores are exact (ids comparable)
    i_all = (np.clip(np.rint(rng.normal(size=(B, N, di)) * 32), -128, 128) / 32).astype(np.float32)
    say("[append] fill 2304 cells in chunks, then the path")
    Kq = torch.zeros((B, N, Hkv, D), dtype=torch.int8, device="cuda")
    Vq = torch.zeros_like(Kq)
    Ksc = torch.zeros((B, N, Hkv, D // 32), dtype=torch.float16, device="cuda")
    Vsc = torch.zeros_like(Ksc)
    Kix = torch.zeros((B, N, di), dtype=torch.float16, device="cuda")
    kd, vd, idd = (torch.from_numpy(a).cuda() for a in (k_all, v_all, i_all))
    pos = 0
    for T in (1, 7, 256, 1000, 1040):           # appends of varying size
        d = qsa.append_desc(batch=B, T=T, n_cells=N, pos0=pos, Hkv=Hkv, D=D, d_idx=di)
        qsa.qsa_kv_append(d, kd[:, pos:pos + T].contiguous(), vd[:, pos:pos + T].contiguous(),
                          idd[:, pos:pos + T].contiguous(), Kq, Ksc, Vq, Vsc, Kix)
        pos += T
    assert pos == N
    torch.cuda.synchronize()
    zero = np.zeros((B, N, Hkv, D), np.int8)
    zs = np.zeros((B, N, Hkv, D // 32), np.uint16)
    rK, rKs, rV, rVs, rI = orc.kv_append(k_all, v_all, i_all, zero, zs, zero, zs,
                                         np.zeros((B, N, di), np.uint16), pos0=0)
    assert np.array_equal(Kq.cpu().numpy(), rK) and np.array_equal(Vq.cpu().numpy(), rV)
    assert np.array_equal(Ksc.cpu().numpy().view(np.uint16), rKs)
    assert np.array_equal(Vsc.cpu().numpy().view(np.uint16), rVs)
    assert np.array_equal(Kix.cpu().numpy().view(np.uint16), rI)
    inp.update(Kq=rK, Ksc=rKs.view(np.float16), Vq=rV, Vsc=rVs.view(np.float16),
               K_idx=rI.view(np.float16))
    res = run_gpu(inp, dev=dict(q_idx=torch.from_numpy(inp["q_idx"]).cuda(), K_idx=Kix,
                                q=torch.from_numpy(inp["q"]).cuda(), Kq=Kq, Ksc=Ksc, Vq=Vq,
                                Vsc=Vsc))
    ref = orc.run(inp, P=4, scale=1.0 / math.sqrt(D))
    assert_ids_equal(res["ids"], res["n_sel"], ref["ids"], ref["n_sel"])
    assert_out_close(res["out"], ref["out"])
