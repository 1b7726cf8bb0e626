"""The binding's size checks (CPU): every call rejects a tensor that holds
fewer bytes than its descriptor addresses, and a tensor that is not on the
GPU, before the library sees the call -- so a short buffer can never be read
or written past its end by a kernel."""
import pytest
import torch

import top_sparse_attention_score_amd as qsa
from top_sparse_attention_score_amd import qsa as binding


def _shapes(B=4, T=1, N=512, di=64, cap=131, Hq=4, Hkv=1, D=64, P=4):
    idesc = qsa.index_desc(batch=B, T=T, n_cells=N, d_idx=di, k=128, pos0=N - 1,
                           dense_max=131, ids_cap=cap)
    adesc = qsa.attn_desc(batch=B, T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, ids_cap=cap, n_cells=N)
    pdesc = qsa.append_desc(batch=B, T=T, n_cells=N, pos0=N - 1, Hkv=Hkv, D=D, d_idx=di)
    t = dict(
        k_new=torch.zeros((B, T, Hkv, D)), v_new=torch.zeros((B, T, Hkv, D)),
        kidx_new=torch.zeros((B, T, di)),
        Kq=torch.zeros((B, N, Hkv, D), dtype=torch.int8),
        Ksc=torch.zeros((B, N, Hkv, D // 32), dtype=torch.float16),
        Vq=torch.zeros((B, N, Hkv, D), dtype=torch.int8),
        Vsc=torch.zeros((B, N, Hkv, D // 32), dtype=torch.float16),
        K_idx=torch.zeros((B, N, di), dtype=torch.float16),
        q_idx=torch.zeros((B, T, di), dtype=torch.float16),
        q=torch.zeros((B, T, Hq, D)), gate=torch.zeros((B, T, Hq, D)),
        ids=torch.zeros((B, T, cap), dtype=torch.int32),
        n_sel=torch.zeros((B, T), dtype=torch.int32), out=torch.zeros((B, T, Hq, D)))
    t["ws"] = torch.zeros(-(-qsa.qsa_step_workspace(idesc, adesc) // 4), dtype=torch.int32)
    return pdesc, idesc, adesc, t


ORDER = ("k_new", "v_new", "kidx_new", "Kq", "Ksc", "Vq", "Vsc", "K_idx", "q_idx", "q", "gate",
         "ids", "n_sel", "out", "ws")


@pytest.mark.parametrize("short", ORDER)
def test_step_rejects_each_short_tensor(short):
    pdesc, idesc, adesc, t = _shapes()
    t[short] = t[short].reshape(-1)[:-1].clone()  # a buffer one element short
    with pytest.raises(qsa.QsaError, match="the call addresses"):
        qsa.qsa_step(pdesc, idesc, adesc, *(t[k] for k in ORDER))


def test_full_size_host_tensors_are_rejected_as_not_on_the_gpu():
    pdesc, idesc, adesc, t = _shapes()
    with pytest.raises(qsa.QsaError, match="not a GPU tensor"):
        qsa.qsa_step(pdesc, idesc, adesc, *(t[k] for k in ORDER))


def test_strided_cache_views_are_measured_to_the_end_of_their_buffer():
    """A scale region that is a view into one cell record is accepted when
    the record buffer reaches the last byte of the last cell's V scales (the
    record's 64 padding bytes after them are not needed), and rejected one
    byte short of it.
    (The check measures a tensor's storage from its data pointer on: the
    bytes a kernel can address without leaving the allocation.)"""
    B, N, Hkv, D = 2, 64, 2, 256
    rec = 1152
    strides = {f"{n}_cell_stride": rec for n in ("kq", "ksc", "vq", "vsc")}
    strides.update({f"{n}_batch_stride": rec * N for n in ("kq", "ksc", "vq", "vsc")})
    adesc = qsa.attn_desc(batch=B, T=1, Hq=24, Hkv=Hkv, D=D, P=4, ids_cap=2051, n_cells=N,
                          strides=strides)
    buf = torch.zeros(B * N * rec, dtype=torch.int8)
    views = (buf[0:], buf[1024:], buf[512:], buf[1056:])
    binding._check_cache(adesc, *views)   # sizes only: accepted
    short = buf[:-(rec - 1088) - 1].clone()
    views = (short[0:], short[1024:], short[512:], short[1056:])
    with pytest.raises(qsa.QsaError, match="Vsc: tensor holds"):
        binding._check_cache(adesc, *views)


def test_each_call_checks_sizes():
    pdesc, idesc, adesc, t = _shapes()
    def cut(x):  # a buffer one element shorter (a slice would keep the whole storage)
        return x.reshape(-1)[:-1].clone()

    q_short = cut(t["q"])
    part = torch.zeros(qsa.qsa_partials_floats(adesc))
    calls = [
        lambda: qsa.qsa_index_topk(idesc, cut(t["q_idx"]), t["K_idx"], t["ids"],
                                   t["n_sel"], t["ws"]),
        lambda: qsa.qsa_index_topk_noalloc(idesc, t["q_idx"], cut(t["K_idx"]), t["ids"],
                                           t["n_sel"]),
        lambda: qsa.qsa_attend(adesc, q_short, t["Kq"], t["Ksc"], t["Vq"], t["Vsc"], t["ids"],
                               t["n_sel"], part),
        lambda: qsa.qsa_attend(adesc, t["q"], t["Kq"], t["Ksc"], t["Vq"], t["Vsc"], t["ids"],
                               t["n_sel"], cut(part)),
        lambda: qsa.qsa_merge(adesc, part, cut(t["out"])),
        lambda: qsa.qsa_merge_gated(adesc, part, cut(t["gate"]), t["out"]),
        lambda: qsa.qsa_attend_merge(adesc, t["q"], t["Kq"], t["Ksc"], cut(t["Vq"]), t["Vsc"],
                                     t["ids"], t["n_sel"], None, t["out"]),
        lambda: qsa.qsa_kv_append(pdesc, t["k_new"], cut(t["v_new"]), t["kidx_new"], t["Kq"],
                                  t["Ksc"], t["Vq"], t["Vsc"], t["K_idx"]),
        lambda: qsa.qsa_decode_window(pdesc, idesc, adesc, *(t[k] for k in ORDER[:-2]),
                                      cut(t["out"]), t["ws"]),
        lambda: qsa.StepCall(pdesc, idesc, adesc, *(t[k] for k in ORDER[:-1]),
                             t["ws"][:1].clone()),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(qsa.QsaError, match="the call addresses"):
            call()
