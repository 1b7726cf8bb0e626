"""GPU tests of qsa_attend_merge: attention with the chunk merge and the
output gate fused into one kernel (P in {1, 2, 4}).

Its output must equal qsa_attend followed by qsa_merge_gated bit for bit
(same partial values, same merge sequence), and therefore meet the oracle
bounds wherever the two calls do.  Cases cover every supported split count,
fp32 and fp16 queries/outputs, gates of both dtypes and none, grid padding
(token counts that are not a multiple of the four items of a workgroup),
empty chunks (rows with fewer kept cells than chunks, and none), head
groups that need one, two and three staging rounds, and the cell-interleaved
cache layout."""
import math

import numpy as np
import pytest
import torch

import top_sparse_attention_score_amd as qsa
from datagen import make_inputs, scattered_ids
from tests.gpu_util import assert_ids_equal, assert_out_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


def _gate(inp, seed):
    rng = np.random.default_rng(seed)
    gdt = np.float16 if inp["q"].dtype == np.float16 else np.float32
    g = (rng.normal(size=inp["q"].shape) * 3).astype(gdt)
    g.reshape(-1)[:4] = (0.0, 40.0, -40.0, -5.0)
    return g


def _fused_and_two_call(inp, *, P, gate=None, ids=None, n_sel=None, strides=None, dev=None):
    """Runs the index (unless ids are given), then both the fused call and
    the two calls on the same ids; returns (fused out, two-call out, path)."""
    path = qsa.path_for(inp, P=P, strides=strides)
    dev = qsa.to_device(inp) if dev is None else dev
    if ids is None:
        path.index(dev["q_idx"], dev["K_idx"])
        ids_t, nsel_t = path.ids, path.n_sel
    else:
        ids_t, nsel_t = torch.from_numpy(ids).cuda(), torch.from_numpy(n_sel).cuda()
    g = None if gate is None else torch.from_numpy(np.ascontiguousarray(gate)).cuda()
    path.attend(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"], ids=ids_t, n_sel=nsel_t)
    path.merge(gate=g)
    torch.cuda.synchronize()
    two = path.out.cpu().numpy().copy()
    path.out.fill_(float("nan"))
    path.attend_merge(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"], gate=g, ids=ids_t,
                      n_sel=nsel_t)
    torch.cuda.synchronize()
    fused = path.out.cpu().numpy().copy()
    return fused, two, path


def _assert_bit_equal(fused, two):
    if not np.array_equal(_bits(fused), _bits(two)):
        bad = np.argwhere(_bits(fused) != _bits(two))
        raise AssertionError(f"fused output differs from the two calls at {len(bad)} "
                             f"elements, first {bad[:3].tolist()}")


PROMPT_SMALL = dict(T=64, N=4096, di=128, k=256, dense_max=259, Hq=24, Hkv=2, D=256, P=1,
                    q_dtype="f16", out_dtype="f16", heavy_tail=False)


@pytest.mark.parametrize("P", [1, 2, 4])
@pytest.mark.parametrize("cfg,batch,gated", [
    ("tiny", 3, True), ("tiny", 5, False), ("decode", 3, True), ("decode", 2, False),
    ("prompt_small", 1, True), ("prompt_small", 1, False)])
def test_fused_equals_two_calls(cfg, batch, gated, P):
    c = PROMPT_SMALL if cfg == "prompt_small" else cfg
    inp = make_inputs(c, seed=410 + batch + 7 * P, batch=batch)
    say(f"[attend_merge] {cfg} B={batch} T={inp['T']} P={P} gate={gated}")
    gate = _gate(inp, 411) if gated else None
    fused, two, _ = _fused_and_two_call(inp, P=P, gate=gate)
    _assert_bit_equal(fused, two)


@pytest.mark.parametrize("G,D", [(1, 64), (8, 64), (16, 64), (2, 256), (16, 256)])
def test_fused_head_groups(G, D):
    """One, two and three staging rounds of the in-LDS merge (7 heads of
    D + 4 floats per round)."""
    cfg = dict(T=3, N=1024, di=64, k=128, dense_max=131, Hq=2 * G, Hkv=2, D=D, P=4,
               q_dtype="f32", out_dtype="f32", heavy_tail=False)
    inp = make_inputs(cfg, seed=420 + G, batch=2)
    say(f"[attend_merge] G={G} D={D}")
    for P in (1, 2, 4):
        fused, two, _ = _fused_and_two_call(inp, P=P, gate=_gate(inp, 421))
        _assert_bit_equal(fused, two)


def test_fused_empty_chunks_and_empty_rows():
    """Rows with fewer kept cells than chunks (empty chunks) and rows with
    none (all chunks empty: the output is 0)."""
    inp = make_inputs("decode", seed=430, batch=2, T=3, N=4096)
    ids, n_sel = scattered_ids(seed=431, batch=2, T=3, N=4096, cap=inp["cap"],
                               pos0=inp["pos0"], n_max=2048)
    n_sel[0, 0] = 0
    n_sel[0, 1] = 1
    n_sel[0, 2] = 3
    n_sel[1, 0] = 2
    n_sel[1, 1] = 5
    ids[n_sel[..., None] <= np.arange(ids.shape[-1])] = -1
    for P in (1, 2, 4):
        fused, two, _ = _fused_and_two_call(inp, P=P, gate=_gate(inp, 432), ids=ids, n_sel=n_sel)
        _assert_bit_equal(fused, two)
        assert np.all(fused[0, 0] == 0), "a row without kept cells merges to 0"


def test_fused_interleaved_layout():
    """The cell-interleaved cache record (both heads' K codes, V codes, K
    scales, V scales in one row per cell) through strided views."""
    inp = make_inputs("decode", seed=440, batch=2)
    B, N, Hkv, D = 2, inp["N"], inp["Hkv"], inp["D"]
    dev = qsa.to_device(inp)
    rec = Hkv * D * 2 + Hkv * (D // 32) * 4
    buf = torch.empty((B, N, rec), dtype=torch.uint8, device="cuda")
    kc, vc = Hkv * D, 2 * Hkv * D
    ks = vc + Hkv * (D // 32) * 2
    buf[:, :, :kc] = dev["Kq"].view(torch.uint8).reshape(B, N, kc)
    buf[:, :, kc:vc] = dev["Vq"].view(torch.uint8).reshape(B, N, kc)
    buf[:, :, vc:ks] = dev["Ksc"].view(torch.uint8).reshape(B, N, -1)
    buf[:, :, ks:] = dev["Vsc"].view(torch.uint8).reshape(B, N, -1)
    flat = buf.reshape(-1)
    view = dict(Kq=flat[0:].view(torch.int8), Vq=flat[kc:].view(torch.int8),
                Ksc=flat[vc:], Vsc=flat[ks:])
    dev2 = dict(dev, **view)
    strides = {f"{n}_cell_stride": rec for n in ("kq", "ksc", "vq", "vsc")}
    strides.update({f"{n}_batch_stride": rec * N for n in ("kq", "ksc", "vq", "vsc")})
    fused, two, _ = _fused_and_two_call(inp, P=4, gate=_gate(inp, 441), strides=strides,
                                        dev=dev2)
    ref_fused, _, _ = _fused_and_two_call(inp, P=4, gate=_gate(inp, 441))
    _assert_bit_equal(fused, two)
    _assert_bit_equal(fused, ref_fused)


@pytest.mark.parametrize("cfg,batch", [("tiny", 3), ("decode", 2)])
def test_fused_against_oracle(orc, cfg, batch):
    """The fused call against the double-precision oracle (ids bit-exact,
    gated output within the workload's bounds)."""
    inp = make_inputs(cfg, seed=450 + batch, batch=batch)
    gate = _gate(inp, 451)
    fused, _, path = _fused_and_two_call(inp, P=inp["P"], gate=gate)
    ref = orc.run(inp, P=inp["P"], scale=1.0 / math.sqrt(inp["D"]))
    want = orc.merge_gated(ref["pm"], ref["pl"], ref["po"], gate)
    assert_ids_equal(path.ids.cpu().numpy(), path.n_sel.cpu().numpy(), ref["ids"], ref["n_sel"])
    assert_out_close(fused.astype(np.float64), want, "fused gated out")


def test_fused_rejects_unsupported_splits():
    """P outside {1, 2, 4} and the vector kernel are rejected before
    anything is enqueued."""
    inp = make_inputs("tiny", seed=460, batch=1)
    dev = qsa.to_device(inp)
    for P in (3, 8, 16):
        path = qsa.path_for(inp, P=P)
        with pytest.raises(qsa.QsaError, match="unsupported"):
            path.attend_merge(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"])
    path = qsa.path_for(inp, P=4, algo=qsa.QSA_ATTEND_VECTOR)
    with pytest.raises(qsa.QsaError, match="unsupported"):
        path.attend_merge(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"])
