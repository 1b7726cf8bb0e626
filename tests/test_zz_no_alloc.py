"""qsa_index_topk_noalloc -- the index call whose workspace is the library's
fixed per-GPU device array -- against qsa_index_topk with a caller-allocated
workspace, through the C ABI: two calls in a row (the second on a smaller
input, so it starts from the first call's leftovers in the shared array),
then a third on another stream.  Ids and n_sel must be equal bit for bit,
and equal to the oracle's (grid inputs).  A shape whose workspace exceeds
the array is rejected with QSA_ERR_WORKSPACE before anything is enqueued."""
import numpy as np
import pytest
import torch

import top_sparse_attention_score_amd as qsa
from datagen import make_inputs
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _desc(inp):
    return qsa.index_desc(batch=inp["batch"], T=inp["T"], n_cells=inp["N"], d_idx=inp["di"],
                          k=inp["k"], pos0=inp["pos0"], dense_max=inp["dense_max"],
                          ids_cap=inp["cap"])


def _both(orc, inp, stream=None):
    d = _desc(inp)
    q = torch.from_numpy(inp["q_idx"]).cuda()
    K = torch.from_numpy(inp["K_idx"]).cuda()
    B, T, cap = inp["batch"], inp["T"], inp["cap"]
    ws_bytes = qsa.qsa_index_topk_workspace(d)
    assert 0 < ws_bytes <= qsa.QSA_NOALLOC_WORKSPACE_BYTES
    ws = torch.empty(ws_bytes // 4 + 1, dtype=torch.int32, device="cuda")
    ids_a = torch.full((B, T, cap), -7, dtype=torch.int32, device="cuda")
    ns_a = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    ids_b = torch.full((B, T, cap), -9, dtype=torch.int32, device="cuda")
    ns_b = torch.full((B, T), -9, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    qsa.qsa_index_topk(d, q, K, ids_a, ns_a, ws, stream=stream)
    qsa.qsa_index_topk_noalloc(d, q, K, ids_b, ns_b, stream=stream)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b) and torch.equal(ns_a, ns_b)
    r_ids, r_ns = orc.index_topk(inp["q_idx"], inp["K_idx"], k=inp["k"], pos0=inp["pos0"],
                                 dense_max=inp["dense_max"], cap=cap)
    assert np.array_equal(ns_b.cpu().numpy(), r_ns) and np.array_equal(ids_b.cpu().numpy(), r_ids)


def test_noalloc_index_matches_workspace_call(orc):
    # 1: long context, chip-wide select (keys, histograms, candidates in the array)
    big = make_inputs("long", seed=9100, batch=2)
    say("[noalloc] call 1: long, B=2, 262144 cells")
    _both(orc, big)
    # 2: smaller, right after: single-token scan + row select over the leftovers
    small = make_inputs("decode", seed=9101, batch=3, N=16384)
    say("[noalloc] call 2: decode-like, B=3, 16384 cells")
    _both(orc, small)
    # 3: eight draft tokens (MFMA scan), on a side stream
    side = torch.cuda.Stream()
    draft = make_inputs("draft", seed=9102, batch=2, N=20000)
    say("[noalloc] call 3: draft, B=2, 20000 cells, side stream")
    _both(orc, draft, stream=side)


def test_noalloc_rejects_oversized_workspace():
    # inputs of the full size the descriptor names (the binding checks
    # sizes before the library sees the call)
    q = torch.zeros((1, 2048, 128), dtype=torch.float16, device="cuda")
    K = torch.zeros((1, 65536, 128), dtype=torch.float16, device="cuda")
    big = qsa.index_desc(batch=1, T=2048, n_cells=65536, d_idx=128, k=2048, pos0=63488,
                         dense_max=2051, ids_cap=2051)
    assert qsa.qsa_index_topk_workspace(big) > qsa.QSA_NOALLOC_WORKSPACE_BYTES
    ids = torch.empty((1, 2048, 2051), dtype=torch.int32, device="cuda")
    ns = torch.empty((1, 2048), dtype=torch.int32, device="cuda")
    with pytest.raises(qsa.QsaError, match="workspace"):
        qsa.qsa_index_topk_noalloc(big, q, K, ids, ns)
