"""The many-token index path (more than 16 tokens against rows of 16384 to
65536 cells) that never writes the score matrix: a sampled lower bound for
each token's k-th largest key, a score GEMM that keeps only the cells at or
above it, and an exact select among those candidates, with a whole-row
fallback for tokens whose candidate list cannot prove the selection (fewer
than k candidates, or more than the list holds).  Ids and n_sel must equal
the oracle's bit for bit on grid inputs, on the normal path and on both
fallbacks."""
import numpy as np
import pytest
import torch

import top_sparse_attention_score_amd as qsa
from datagen import make_inputs
from tests.gpu_util import assert_ids_equal, say
from tests.oracle_pool import host_threads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _gpu_ids(inp):
    path = qsa.path_for(inp)
    dev = qsa.to_device(inp)
    path.index(dev["q_idx"], dev["K_idx"])
    torch.cuda.synchronize()
    return path.ids.cpu().numpy(), path.n_sel.cpu().numpy()


def _oracle_ids(orc, inp, slice_tokens=8):
    """The oracle's ids over token slices on the host threads."""
    from concurrent.futures import ThreadPoolExecutor
    B, T = inp["q_idx"].shape[:2]
    ids = np.empty((B, T, inp["cap"]), np.int32)
    ns = np.empty((B, T), np.int32)

    def one(job):
        b, t0 = job
        t1 = min(T, t0 + slice_tokens)
        i, n = orc.index_topk(inp["q_idx"][b:b + 1, t0:t1], inp["K_idx"][b:b + 1], k=inp["k"],
                              pos0=inp["pos0"] + t0, dense_max=inp["dense_max"], cap=inp["cap"])
        ids[b, t0:t1], ns[b, t0:t1] = i[0], n[0]

    with ThreadPoolExecutor(host_threads()) as ex:
        list(ex.map(one, [(b, t0) for b in range(B) for t0 in range(0, T, slice_tokens)]))
    return ids, ns


# Many tokens (four 16-token column blocks per workgroup) and 2-16 tokens
# (one column block: the draft's shape), with ragged last blocks.
@pytest.mark.parametrize("N,T,pos0,batch", [(65536, 256, 65280, 1), (65536, 128, 30000, 2),
                                            (40000, 200, 39800, 1), (16384, 64, 16320, 2),
                                            (65536, 8, 65528, 2), (65536, 16, 60000, 1),
                                            (65536, 17, 65000, 1), (30000, 5, 29990, 3),
                                            (16384, 2, 16382, 2)])
def test_fused_index_matches_oracle(orc, N, T, pos0, batch):
    inp = make_inputs("prompt", seed=9300 + T, batch=batch, N=N, T=T, pos0=pos0)
    say(f"[fused index] N={N} T={T} pos0={pos0} B={batch}")
    ids, ns = _gpu_ids(inp)
    r_ids, r_ns = _oracle_ids(orc, inp)
    assert_ids_equal(ids, ns, r_ids, r_ns)


def _sample_cells(span: int, n: int = 2048) -> np.ndarray:
    """Cells the library samples for the candidate bound (spread evenly, a
    hashed offset inside each stride), to plant a case that defeats it."""
    stride = max(1, span // n)
    s = np.arange(n, dtype=np.uint64)
    off = (((s * 0x9E3779B1) & 0xFFFFFFFF) >> 16) % stride
    return (s * stride + off).astype(np.int64)


@pytest.mark.parametrize("T", [64, 8])
def test_fused_index_fallbacks(orc, T):
    """Problem 0: the first quarter of the tokens have a zero index query
    (every score equal), the second quarter see scores from two values (half
    the row ties at the top): their candidate lists overflow.  Problem 1:
    1000 sampled cells are planted above all others, so the sampled bound
    keeps fewer than k candidates.  Problem 2: four score values, a large
    exact tie at the k-th inside the candidate list.  The other half of
    problem 0's tokens take the normal path.  T = 64 runs four column blocks
    per workgroup, T = 8 one."""
    N = 65536
    pos0 = N - T
    q1, q2 = T // 4, T // 2
    inp = make_inputs("prompt", seed=9400 + T, batch=3, N=N, T=T, pos0=pos0)
    inp["q_idx"][0, :q1] = 0
    rng = np.random.default_rng(9401)
    inp["q_idx"][0, q1:q2] = 0
    inp["q_idx"][0, q1:q2, 0] = 1.0
    inp["K_idx"][0, :, 0] = np.where(rng.random(N) < 0.5, 1.0, 0.0).astype(np.float16)
    cells = _sample_cells(pos0 + T)
    assert len(np.unique(cells)) == 2048 and cells[:1000].max() <= pos0
    # 1000 of the sampled cells score above every other cell: the sample's
    # ~100th largest key lies among them, so only ~100 cells reach the bound
    inp["K_idx"][1] = np.clip(inp["K_idx"][1], -1, 1)
    inp["q_idx"][1] = np.abs(inp["q_idx"][1])
    planted = cells[:1000]
    inp["K_idx"][1, planted] += np.float16(3.0)
    # Problem 2: scores in {0, 1, 2, 3} (1% at 3, 3% at 2): the candidates
    # (score >= 2, about 2600) fit the list, but the ~1970 tied at 2 share one
    # bin of the candidate histogram, which the select resolves by radix.
    inp["q_idx"][2] = 0
    inp["q_idx"][2, :, 0] = 1.0
    inp["K_idx"][2] = 0
    inp["K_idx"][2, :, 0] = rng.choice(np.array([0.0, 1.0, 2.0, 3.0], np.float16), size=N,
                                       p=[0.5, 0.46, 0.03, 0.01])
    say("[fused index] fallbacks: ties, two-valued scores, planted sample, 4-valued")
    ids, ns = _gpu_ids(inp)
    r_ids, r_ns = _oracle_ids(orc, inp)
    assert_ids_equal(ids, ns, r_ids, r_ns)
    assert np.all(np.isin(planted, r_ids[1, 0, :2048]))


# One token against rows longer than the register select holds (65,537 to
# 262,144 cells): sampled bound, the scan keeping only candidates, exact
# select among them.  The attention shape is shrunk (the index path does not
# read it) to keep the inputs small.
SMALL_KV = dict(Hq=4, Hkv=1, D=64)


@pytest.mark.parametrize("cfg,N,pos0,batch,grid", [
    ("long", 262144, 262143, 2, True),      # the long workload's rows (planted heavy tail)
    ("long", 262144, 262143, 1, False),     # raw fp16 keys
    ("decode", 100000, 99999, 3, True),
    ("decode", 262144, 70000, 1, True),     # visible part of the row only
    ("decode", 131072, 65536, 2, True),     # just past the register select
    ("tiny", 80000, 79999, 2, True),        # d_idx 64, k 128
])
def test_long_row_index_matches_oracle(orc, cfg, N, pos0, batch, grid):
    inp = make_inputs(cfg, seed=9500 + batch, batch=batch, N=N, pos0=pos0, index_grid=grid,
                      **(SMALL_KV if cfg != "tiny" else {}))
    say(f"[long-row index] {cfg} N={N} pos0={pos0} B={batch} grid={grid}")
    ids, ns = _gpu_ids(inp)
    r_ids, r_ns = _oracle_ids(orc, inp)
    if grid:
        assert_ids_equal(ids, ns, r_ids, r_ns)
    else:
        n_diff = _bounded_ids(inp, ids, ns, r_ids, r_ns)
        say(f"[long-row index] raw fp16: {n_diff} ids differ, all within the bound")


def _bounded_ids(inp, ids, ns, r_ids, r_ns):
    """General fp16 keys: an id may differ from the oracle's only for a cell
    whose double score lies within 2 gamma_d max_j sum_i |q_i k_ji| of the
    k-th double score (fp32 summation bound); returns the differing ids."""
    di = inp["q_idx"].shape[-1]
    u = 2.0 ** -24
    g2 = 2.0 * di * u / (1.0 - di * u)
    assert np.array_equal(ns, r_ns)
    n_diff = 0
    for b in range(ids.shape[0]):
        for t in range(ids.shape[1]):
            n = int(ns[b, t])
            kept, want = ids[b, t, :n], r_ids[b, t, :n]
            assert np.all(ids[b, t, n:] == -1) and np.all(np.diff(kept) > 0)
            if np.array_equal(kept, want):
                continue
            nvis = inp["pos0"] + t + 1
            q = inp["q_idx"][b, t].astype(np.float64)
            K = inp["K_idx"][b, :nvis].astype(np.float64)
            sc = K @ q
            slack = g2 * (np.abs(K) @ np.abs(q)).max()
            diff = np.setxor1d(kept, want)
            assert np.abs(sc[diff] - sc[want].min()).max() <= slack
            n_diff += len(diff)
    return n_diff


def test_long_row_fallbacks(orc):
    """Problem 0: a zero index query (every score equal): the candidate list
    overflows and the row is scored and selected whole.  Problem 1: 1000
    sampled cells planted above all others: the bound keeps fewer than k
    candidates.  Problem 2: four score values, a large exact tie at the k-th
    inside the candidate list.  Problem 3 takes the normal path."""
    N = 262144
    pos0 = N - 1
    inp = make_inputs("long", seed=9600, batch=4, N=N, pos0=pos0, **SMALL_KV)
    rng = np.random.default_rng(9601)
    inp["q_idx"][0] = 0
    cells = _sample_cells(pos0 + 1)
    assert len(np.unique(cells)) == 2048 and cells.max() <= pos0
    inp["K_idx"][1] = np.clip(inp["K_idx"][1], -1, 1)
    inp["q_idx"][1] = np.abs(inp["q_idx"][1])
    planted = cells[:1000]
    inp["K_idx"][1, planted] += np.float16(3.0)
    inp["q_idx"][2] = 0
    inp["q_idx"][2, :, 0] = 1.0
    inp["K_idx"][2] = 0
    inp["K_idx"][2, :, 0] = rng.choice(np.array([0.0, 1.0, 2.0, 3.0], np.float16), size=N,
                                       p=[0.5, 0.4925, 0.006, 0.0015])
    say("[long-row index] fallbacks: all equal, planted sample, 4-valued ties")
    ids, ns = _gpu_ids(inp)
    r_ids, r_ns = _oracle_ids(orc, inp)
    assert_ids_equal(ids, ns, r_ids, r_ns)
    assert np.all(np.isin(planted, r_ids[1, 0, :2048]))
