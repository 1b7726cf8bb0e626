"""GPU parity: the HIP path (through the C ABI) against the double-precision
oracle on seeded inputs of the five workloads, the pos0 x ntok sweep of the
pages' bitwise check, attention-only runs on random scattered ids, and the
pages' bit-exact claims (zero padding, exact max, determinism)."""
import math

import numpy as np
import pytest
import torch

from datagen import make_inputs, scattered_ids, sweep_cases
from tests.gpu_util import (assert_ids_equal, assert_out_close, assert_partials_close,
                            run_gpu, say)
from tests.oracle_pool import host_threads, oracle_all_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _oracle_all(orc, inp, P):
    return orc.run(inp, P=P, scale=1.0 / math.sqrt(inp["D"]))


# ------------------------------------------------------------ workloads ---

@pytest.mark.parametrize("algo", ["matrix", "vector"])
@pytest.mark.parametrize("cfg,batch", [("tiny", 3), ("decode", 2), ("draft", 1), ("long", 1)])
def test_workload_parity(orc, cfg, batch, algo):
    inp = make_inputs(cfg, seed=1000 + batch, batch=batch)
    say(f"[parity] {cfg} B={batch} T={inp['T']} N={inp['N']} P={inp['P']} {algo}")
    res = run_gpu(inp, algo=algo)
    ref = _oracle_all(orc, inp, inp["P"])
    assert_ids_equal(res["ids"], res["n_sel"], ref["ids"], ref["n_sel"])
    assert_partials_close(res, ref["pm"], ref["pl"], ref["po"])
    assert_out_close(res["out"], ref["out"])


_PROMPT_REF = {}


def _prompt_reference(orc, inp):
    """The oracle's ids and output for all 2048 tokens of the prompt chunk
    (computed once per module, in parallel slices on the host cores)."""
    if "ref" not in _PROMPT_REF:
        say(f"[parity] prompt: oracle over all {inp['T']} tokens on {host_threads()} threads")
        _PROMPT_REF["ref"] = oracle_all_tokens(orc, inp, P=1,
                                               scale=1.0 / math.sqrt(inp["D"]))
    return _PROMPT_REF["ref"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("algo", ["matrix", "vector"])
def test_prompt_chunk_full(orc, algo):
    """The 2048-token prompt chunk at full size on the GPU against the
    oracle on every token: ids and n_sel bit for bit, the fp16 output of
    every token within tolerance."""
    inp = make_inputs("prompt", seed=1005)
    say(f"[parity] prompt T=2048 N=65536 full size {algo}")
    res = run_gpu(inp, algo=algo)
    ref = _prompt_reference(orc, inp)
    assert_ids_equal(res["ids"], res["n_sel"], ref["ids"], ref["n_sel"])
    assert_out_close(res["out"], ref["out"], "prompt chunk, all tokens")
    worst = max(float(np.abs(res["out"][:, t].astype(np.float64) - ref["out"][:, t]).max())
                for t in range(inp["T"]))
    say(f"[parity] prompt {algo}: worst token max-abs error {worst:.3e}")


def test_pos_sweep(orc):
    """pos0 in {0,1,63,64,512,2047,2048,2050,8192,30000} x ntok in {1,2,4,8}
    on a 32768-cell cache: dense fallback, the 2051 bound and top-k."""
    for pos0, ntok in sweep_cases():
        inp = make_inputs("decode", seed=2000 + pos0 + ntok, N=32768, T=ntok, pos0=pos0)
        say(f"[sweep] pos0={pos0} ntok={ntok}")
        res = run_gpu(inp)
        ref = _oracle_all(orc, inp, inp["P"])
        assert_ids_equal(res["ids"], res["n_sel"], ref["ids"], ref["n_sel"])
        assert_out_close(res["out"], ref["out"], f"pos0={pos0} ntok={ntok}")


@pytest.mark.parametrize("algo", ["matrix", "vector"])
@pytest.mark.parametrize("P", [1, 2, 3, 8, 16, 64])
def test_split_counts(orc, P, algo):
    inp = make_inputs("decode", seed=3000 + P, batch=1)
    say(f"[split] P={P} {algo}")
    res = run_gpu(inp, P=P, algo=algo)
    ref = _oracle_all(orc, inp, P)
    assert_ids_equal(res["ids"], res["n_sel"], ref["ids"], ref["n_sel"])
    assert_partials_close(res, ref["pm"], ref["pl"], ref["po"])
    assert_out_close(res["out"], ref["out"])


@pytest.mark.parametrize("algo", ["matrix", "vector"])
@pytest.mark.parametrize("n_max", [1, 5, 31, 32, 33, 64, 65, 300, 2051])
def test_attend_scattered_ids(orc, n_max, algo):
    """Attention and merge alone on random scattered ids (decoupled from the
    indexer), per the pages' bitwise-check input; chunk lengths straddle the
    32-cell tile of the matrix kernel."""
    inp = make_inputs("decode", seed=4000 + n_max, batch=2, N=32768, T=4, pos0=30000)
    ids, n_sel = scattered_ids(seed=5, batch=2, T=4, N=32768, cap=inp["cap"], pos0=30000,
                               n_max=n_max)
    say(f"[scattered] n_max={n_max} {algo}")
    res = run_gpu(inp, ids=ids, n_sel=n_sel, index=False, algo=algo)
    pm, pl, po = orc.attend(inp["q"], inp["Kq"], inp["Ksc"], inp["Vq"], inp["Vsc"], ids,
                            n_sel, P=inp["P"], scale=1 / 16)
    assert_partials_close(res, pm, pl, po)
    assert_out_close(res["out"], orc.merge(pm, pl, po))


@pytest.mark.parametrize("algo", ["matrix", "vector"])
def test_tiny_fp16_and_gqa_variants(orc, algo):
    """Every supported (G, D) pair with fp32 and fp16 queries on small inputs."""
    for D in (64, 256):
        for G in (1, 2, 4, 8, 12, 16):
            for qd in ("f32", "f16"):
                Hkv = 2 if G <= 8 else 1
                cfg = dict(T=2, N=700, di=64, k=150, dense_max=153, Hq=G * Hkv, Hkv=Hkv,
                           D=D, P=3, q_dtype=qd, out_dtype=qd, heavy_tail=False)
                inp = make_inputs(cfg, seed=G * 10 + D)
                say(f"[variant] D={D} G={G} q={qd} {algo}")
                res = run_gpu(inp, algo=algo)
                ref = _oracle_all(orc, inp, 3)
                assert_ids_equal(res["ids"], res["n_sel"], ref["ids"], ref["n_sel"])
                assert_out_close(res["out"], ref["out"], f"D={D} G={G} {qd}")


def test_tie_stress(orc):
    """40 identical index keys straddle rank 128 of a 512-cell cache: the kept
    ids must give the tie quota to the lowest indices, bit-exactly."""
    inp = make_inputs("tiny", seed=77, batch=2)
    rng = np.random.default_rng(78)
    for b in range(2):
        s = inp["q_idx"][b, 0].astype(np.float64) @ inp["K_idx"][b].astype(np.float64).T
        order = np.lexsort((np.arange(512), -s))
        group = rng.choice(order[100:160], size=40, replace=False)
        inp["K_idx"][b, group] = inp["K_idx"][b, order[128]]
    res = run_gpu(inp)
    ref = _oracle_all(orc, inp, inp["P"])
    assert_ids_equal(res["ids"], res["n_sel"], ref["ids"], ref["n_sel"])
    assert_out_close(res["out"], ref["out"])


def test_all_scores_equal(orc):
    """q_idx = 0: every visible cell scores 0, so top-k is the k lowest ids."""
    inp = make_inputs("decode", seed=79)
    inp["q_idx"][:] = 0
    res = run_gpu(inp)
    assert res["n_sel"][0, 0] == 2048
    assert np.array_equal(res["ids"][0, 0, :2048], np.arange(2048))
    ref = _oracle_all(orc, inp, inp["P"])
    assert_out_close(res["out"], ref["out"])


def test_interleaved_cache_layout(orc):
    """Codes and scales of a cell interleaved in one buffer via the strides
    give the same result as the dense layout."""
    inp = make_inputs("decode", seed=80, batch=2, N=4096)
    B, N, Hkv, D = 2, 4096, 2, 256
    rec = Hkv * D + Hkv * (D // 32) * 2          # 544 bytes: codes, then scales
    buf = {}
    for name, codes, scales in (("K", inp["Kq"], inp["Ksc"]), ("V", inp["Vq"], inp["Vsc"])):
        raw = np.zeros((B, N, rec), dtype=np.uint8)
        raw[:, :, :Hkv * D] = codes.reshape(B, N, -1).view(np.uint8)
        raw[:, :, Hkv * D:] = scales.reshape(B, N, -1).view(np.uint8)
        buf[name] = torch.from_numpy(raw).cuda()
    strides = dict(kq_cell_stride=rec, ksc_cell_stride=rec, vq_cell_stride=rec,
                   vsc_cell_stride=rec, kq_batch_stride=N * rec, ksc_batch_stride=N * rec,
                   vq_batch_stride=N * rec, vsc_batch_stride=N * rec)
    import top_sparse_attention_score_amd as qsa
    dev = qsa.to_device(inp)
    path = qsa.path_for(inp, strides=strides)
    path.index(dev["q_idx"], dev["K_idx"])
    Kb, Vb = buf["K"], buf["V"]
    path.attend(dev["q"], Kb, Kb[:, :, Hkv * D:], Vb, Vb[:, :, Hkv * D:])
    path.merge()
    torch.cuda.synchronize()
    dense = run_gpu(inp)
    assert np.array_equal(path.out.cpu().numpy(), dense["out"])
    ref = _oracle_all(orc, inp, inp["P"])
    assert_out_close(dense["out"], ref["out"])


# ------------------------------------------------ the pages' bit claims ---

@pytest.mark.parametrize("algo", ["matrix", "vector"])
def test_padding_beyond_n_sel_is_ignored(algo):
    """Entries past n_sel never change the partials (an absent cell adds
    p = 0): garbage padding gives bitwise-identical partials and output."""
    inp = make_inputs("decode", seed=81, batch=2, N=16384, T=3, pos0=16000)
    ids, n_sel = scattered_ids(seed=9, batch=2, T=3, N=16384, cap=inp["cap"], pos0=16000,
                               n_max=1000)
    a = run_gpu(inp, ids=ids, n_sel=n_sel, index=False, algo=algo)
    ids2 = ids.copy()
    rng = np.random.default_rng(10)
    for b in range(2):
        for t in range(3):
            n = n_sel[b, t]
            ids2[b, t, n:] = rng.integers(0, 16384, size=ids2.shape[-1] - n)
    b_ = run_gpu(inp, ids=ids2, n_sel=n_sel, index=False, algo=algo)
    for key in ("pm", "pl", "po", "out"):
        assert a[key].tobytes() == b_[key].tobytes(), key


@pytest.mark.parametrize("algo", ["matrix", "vector"])
def test_run_to_run_determinism(algo):
    inp = make_inputs("draft", seed=82, N=16384)
    a = run_gpu(inp, algo=algo)
    b = run_gpu(inp, algo=algo)
    for key in ("ids", "n_sel", "pm", "pl", "po", "out"):
        assert a[key].tobytes() == b[key].tobytes(), key


@pytest.mark.parametrize("algo", ["matrix", "vector"])
def test_position_zero_is_exact(algo):
    """A token at position 0 keeps only cell 0 and its output is that cell's
    dequantised V row, bit for bit (exp(0) = 1, the weight 1 times an fp16
    scale and an int8 code is exact in either kernel, v / 1 = v)."""
    inp = make_inputs("decode", seed=83, batch=2, N=64, T=1, pos0=0)
    res = run_gpu(inp, algo=algo)
    assert np.all(res["n_sel"] == 1) and np.all(res["ids"][:, :, 0] == 0)
    v = (inp["Vq"][:, 0].astype(np.float64) *
         np.repeat(inp["Vsc"][:, 0].astype(np.float64), 32, axis=-1)).astype(np.float32)
    G = inp["Hq"] // inp["Hkv"]
    for h in range(inp["Hq"]):
        assert res["out"][:, 0, h].tobytes() == v[:, h // G].tobytes()


@pytest.mark.parametrize("algo", ["matrix", "vector"])
def test_chunk_max_is_exact_max_of_logits(algo):
    """The partial max of a one-cell chunk is that cell's logit, and the max
    of a chunk equals the max over its one-cell chunks bit for bit."""
    inp = make_inputs("decode", seed=84, batch=1, N=4096, T=1, pos0=4095, k=64,
                      dense_max=67)
    one = run_gpu(inp, P=64, algo=algo)          # 64 ids -> 64 one-cell chunks
    whole = run_gpu(inp, P=1, algo=algo)
    assert np.all(one["pl"] == 1.0)
    assert whole["pm"][..., 0].tobytes() == one["pm"].max(axis=-1).tobytes()


@pytest.mark.parametrize("algo", ["matrix", "vector"])
@pytest.mark.parametrize("cfg,batch", [("decode", 2), ("draft", 1), ("tiny", 4)])
def test_fp32_level_precision(orc, cfg, batch, algo):
    """Both attention kernels keep fp32-level accuracy, far inside the
    workload tolerance: fp32 accumulation of <= 2048 exact products gives a
    relative error of order 2^-24 * sqrt(2048) ~ 3e-6, so rel-L2 <= 1e-5.
    A lost lo half of a split fp16 operand in the matrix kernel would show
    as ~2^-11 (5e-4) relative error and fail this."""
    inp = make_inputs(cfg, seed=77, batch=batch)
    say(f"[precision] {cfg} B={batch} {algo}")
    res = run_gpu(inp, algo=algo)
    ref = _oracle_all(orc, inp, inp["P"])
    diff = res["out"].astype(np.float64) - ref["out"]
    rel = np.linalg.norm(diff) / np.linalg.norm(ref["out"])
    assert rel <= 1e-5, rel
    fin = np.isfinite(ref["pm"])
    assert np.abs(res["pm"].astype(np.float64)[fin] - ref["pm"][fin]).max() <= 1e-5


@pytest.mark.parametrize("cfg,batch", [("decode", 2), ("tiny", 3), ("prompt_small", 1)])
def test_gated_merge(orc, cfg, batch):
    """qsa_merge_gated: the merged output times sigmoid(gate) elementwise,
    with an fp32 gate (fp32 q) or an fp16 gate (fp16 q, fp16 output)."""
    if cfg == "prompt_small":
        cfg = dict(T=64, N=4096, di=128, k=256, dense_max=259, Hq=24, Hkv=2, D=256, P=1,
                   q_dtype="f16", out_dtype="f16", heavy_tail=False)
    inp = make_inputs(cfg, seed=95, batch=batch)
    rng = np.random.default_rng(96)
    gdt = np.float16 if inp["q"].dtype == np.float16 else np.float32
    gate = (rng.normal(size=inp["q"].shape) * 3).astype(gdt)
    gate.reshape(-1)[:4] = (0.0, 40.0, -40.0, -5.0)
    say(f"[gate] {inp['T']} tokens, gate {gdt.__name__}")
    res = run_gpu(inp, gate=gate)
    ref = _oracle_all(orc, inp, inp["P"])
    want = orc.merge_gated(ref["pm"], ref["pl"], ref["po"], gate)
    assert_ids_equal(res["ids"], res["n_sel"], ref["ids"], ref["n_sel"])
    assert_out_close(res["out"], want, "gated out")


def test_graph_replay_matches_eager(orc):
    """The whole step (append -> index_topk -> attend -> gated merge) captured
    in a HIP graph: every replay, with eager work and synchronisations in
    between, gives bitwise the eager result (the path records no memset)."""
    import top_sparse_attention_score_amd as qsa
    inp = make_inputs("decode", seed=97, batch=1)
    dev = qsa.to_device(inp)
    rng = np.random.default_rng(98)
    B, T, Hkv, D, di = 1, inp["T"], inp["Hkv"], inp["D"], inp["di"]
    k_new = torch.from_numpy(rng.normal(size=(B, T, Hkv, D)).astype(np.float32)).cuda()
    v_new = torch.from_numpy(rng.normal(size=(B, T, Hkv, D)).astype(np.float32)).cuda()
    i_new = torch.from_numpy(rng.normal(size=(B, T, di)).astype(np.float32)).cuda()
    dev["gate"] = torch.from_numpy(rng.normal(size=inp["q"].shape).astype(np.float32)).cuda()
    adesc = qsa.append_desc(batch=B, T=T, n_cells=inp["N"], pos0=inp["pos0"], Hkv=Hkv, D=D,
                            d_idx=di)
    path = qsa.path_for(inp)
    side = torch.cuda.Stream()

    def step(stream):
        qsa.qsa_kv_append(adesc, k_new, v_new, i_new, dev["Kq"], dev["Ksc"], dev["Vq"],
                          dev["Vsc"], dev["K_idx"], stream=stream)
        path.run(dev, stream=stream)

    step(None)
    torch.cuda.synchronize()
    eager = path.out.clone()
    ids = path.ids.clone()
    g = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        path.out.zero_()
        path.ids.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(path.out, eager), rep
        assert torch.equal(path.ids, ids), rep
        step(None)                      # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("case", ["all_equal", "few_values"])
def test_chip_wide_select_ties(orc, case):
    """Rows longer than 65536 cells take the chip-wide select.  With every
    score equal (q_idx = 0) the threshold bin holds all cells and the pivot
    kernel streams the keys (more candidates than its list); with scores
    from a few distinct values the threshold bin is a large exact tie.
    Both must give the lowest-index rule bit for bit."""
    cfg = dict(T=2, N=70000, di=64, k=2048, dense_max=2051, Hq=4, Hkv=1, D=64, P=4,
               q_dtype="f32", out_dtype="f32", heavy_tail=False)
    inp = make_inputs(cfg, seed=101, batch=2)
    if case == "all_equal":
        inp["q_idx"][:] = 0
    else:
        rng = np.random.default_rng(102)
        vals = np.array([-1.0, 0.0, 0.5, 2.0], np.float16)
        inp["K_idx"][:] = 0
        inp["K_idx"][..., 0] = vals[rng.integers(0, 4, size=inp["K_idx"].shape[:2])]
        inp["q_idx"][:] = 0
        inp["q_idx"][..., 0] = 1.0
    say(f"[chip-wide select] {case}")
    res = run_gpu(inp)
    ref = _oracle_all(orc, inp, inp["P"])
    assert_ids_equal(res["ids"], res["n_sel"], ref["ids"], ref["n_sel"])
    assert_out_close(res["out"], ref["out"])
    if case == "all_equal":
        for t in range(inp["T"]):
            assert np.array_equal(res["ids"][:, t, :2048], np.tile(np.arange(2048), (2, 1)))


@pytest.mark.parametrize("cfg,batch", [("decode", 512), ("draft", 32), ("long", 16)])
def test_bench_launch_configuration(orc, cfg, batch):
    """The batch sizes bench.py times, built the way it builds them (a few
    distinct seeded problems tiled over the batch): every replica's ids equal
    its problem's oracle ids bit for bit and its output is within tolerance."""
    import top_sparse_attention_score_amd as qsa
    nd = min(4, batch)
    base = make_inputs(cfg, seed=103, batch=nd)
    reps = batch // nd
    dev = {}
    for key in ("q_idx", "K_idx", "q", "Kq", "Ksc", "Vq", "Vsc"):
        t = torch.from_numpy(base[key]).cuda()
        dev[key] = t.repeat((reps,) + (1,) * (t.dim() - 1)).contiguous()
    inp = dict(base)
    inp["batch"] = batch
    say(f"[bench config] {cfg} B={batch} ({nd} distinct problems)")
    path = qsa.path_for(inp)
    path.run(dev)
    torch.cuda.synchronize()
    ref = _oracle_all(orc, base, base["P"])
    ids, n_sel, out = path.ids.cpu().numpy(), path.n_sel.cpu().numpy(), path.out.cpu().numpy()
    for b in range(batch):
        d = b % nd
        assert_ids_equal(ids[b], n_sel[b], ref["ids"][d], ref["n_sel"][d])
        assert_out_close(out[b], ref["out"][d], f"replica {b}")
