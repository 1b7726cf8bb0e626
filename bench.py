"""Throughput benchmark of the QSA hot path on one MI355X.

One step = append -> index_topk -> attend -> gated merge over a batch of B
independent problems (seeded synthetic caches already resident in HBM): the
step's T new tokens are quantised into their cells of the cache, then
selected from and attended to, and the merged output is gated.  The step is
one qsa_step call, which runs those four calls in the fewest kernel launches
the shape allows (the append inside the decode scan/select kernel, the merge
inside the attention kernel when P is 1, 2 or 4); --merge separate times the
four calls one by one instead.
The default workload is the decode step (1 token, 24 x 256 query heads,
2 KV heads, 8192 cached cells, index dim 128, top-2048) over B = 512
independent caches, so the working set (~5.4 GB) is far larger than the
256 MB last-level cache and every step streams from HBM.  At 512 problems
each of the step's two kernels runs two rounds of workgroups over the
chip, which hides most of one round's ramp-up and drain (256 problems, one
round each, reach ~4.5% less).

Timing: after the W warm-up steps (and the probes), untimed steps continue
until about 0.2 s of GPU time has passed (this GPU's clocks settle under a sustained HBM load
only after some tens of milliseconds).  The K timed steps then run back to
back between two HIP events on the launch stream (nothing else is enqueued
between them); four more such blocks give the median/min/max over rounds.  A separate pass of the same
calls one by one, with an event between stages, gives the per-stage
breakdown (each event adds a few microseconds of its own), and the
roofline's kernel time is the average of ten back-to-back launches of the
dominant stage.

Prints one JSON line: metric/value (kept KV cells attended per second),
stage times, algorithmic HBM bytes and flops, the roofline of the dominant
kernel, and the oracle's throughput on a bounded sample of the same
workload on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selected KV cells attended/sec + achieved HBM GB/s (% of 8 TB/s), 1 MI355X"
HBM_PEAK_GBS = 8000.0
# fp32 FMA peak without packed-fp32 instructions: 256 CUs x 4 SIMDs x 16 lanes
# x 2 flop x 2.4 GHz.
FP32_VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12   # 78.6

# Split count of the single-problem latency run where the workload leaves it
# free (decode: one problem has only Hkv * P waves of attention, so more
# chunks); the others keep the split their definition fixes.
LATENCY_P = {"decode": 32}

WORKLOADS = {
    # name: (datagen config, default batch, description)
    "decode": ("decode", 512, "decode step: 1 token, 24x256 q heads, 2 KV heads, 8192 cells, "
                              "index dim 128, top-2048, int8 KV + fp16 scale per 32"),
    "draft": ("draft", 32, "draft batch: 8 tokens, 24x256 q heads, 2 KV heads, 65536 cells, "
                           "top-2048 per token"),
    "long": ("long", 16, "long context: 1 token, 24x256 q heads, 2 KV heads, 262144 cells, "
                         "top-2048, planted heavy-tail index scores"),
    "prompt": ("prompt", 1, "prompt chunk: 2048 tokens vs 65536 cells, fp16 q/out, "
                            "top-2048 per token"),
    "tiny": ("tiny", 1024, "tiny: 1 token, 4x64 q heads, 1 KV head, 512 cells, top-128"),
}


def algorithmic_bytes(p: dict, B: int, n_sel_total: int) -> dict:
    """Bytes the method must move per step (no reuse across tokens): the new
    tokens' fp32 K/V/index rows in and their codes, scales and fp16 index
    keys out; index keys of every visible cell once per call (when any token
    selects); the kept cells' K/V codes and scales once per token, q, ids,
    output."""
    T, N, di, Hq, Hkv, D, k = p["T"], p["N"], p["di"], p["Hq"], p["Hkv"], p["D"], p["k"]
    append = B * T * (2 * Hkv * D * 4 + di * 4 + 2 * Hkv * (D + (D // 32) * 2) + di * 2)
    pos0 = p.get("pos0", N - T)
    nvis_max = pos0 + T
    qbytes = 2 if p["q_dtype"] == "f16" else 4
    obytes = 2 if p["out_dtype"] == "f16" else 4
    selects = nvis_max > p["dense_max"] and nvis_max > k
    index = B * (nvis_max * di * 2 + T * di * 2) if selects else 0
    per_cell = Hkv * (D + (D // 32) * 2) * 2          # K and V codes + scales
    attend = n_sel_total * (per_cell + 4) + B * T * Hq * D * qbytes
    out = B * T * Hq * D * (obytes + qbytes)              # output and its gate
    return dict(append=append, index=index, attend=attend, out=out,
                total=append + index + attend + out)


def attend_flops(p: dict, n_sel_total: int) -> float:
    return float(n_sel_total) * p["Hq"] * p["D"] * 4      # QK + PV FMAs, 2 flop each


# Source file of each attend kernel family (its hash gates profiled traffic).
ATTEND_SOURCES = {"matrix": "qsa_attend_mma.hip", "vector": "qsa_attend.hip"}
ATTEND_KERNELS = {"matrix": "k_attend_mma", "vector": "k_attend",
                  "matrix_merge": "k_attend_merge_mma", "matrix_mch": "k_attend_mch_mma"}
# Headers whose code the attend kernels compile in (also hashed).
ATTEND_HEADERS = ("qsa_device.h", "qsa_mma.h", "qsa_attend_mma.h", "qsa_merge.h")
# Source and headers of the index kernels (their hash gates profiled index
# traffic).
INDEX_FILES = ("qsa_index.hip", "qsa_select.h", "qsa_device.h", "qsa_mma.h")


def source_hash(files) -> str:
    import hashlib
    csrc = os.path.join(ROOT, "top_sparse_attention_score_amd", "csrc")
    return hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read()
                                   for f in files)).hexdigest()[:16]


def _profile_fields(workload: str, B: int, P: int, algo: str, layout: str) -> dict:
    kern = ATTEND_KERNELS[algo]
    tag = "" if layout == "dense" else f"_{layout}"
    path = os.path.join(ROOT, "profiles", f"{kern}_{workload}_b{B}_P{P}{tag}.md")
    fields = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith(("|", "#", "`")):
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    return fields


def profiled_index_traffic(workload: str, B: int, P: int, algo: str, layout: str):
    """HBM bytes of one index_topk call (all its kernels) from the same
    committed summary; None if absent or the index sources changed."""
    f = _profile_fields(workload, B, P, algo, layout)
    if f.get("index_source_sha256_16") != source_hash(INDEX_FILES):
        return None
    try:
        return int(f["index_read_bytes_per_call"]) + int(f["index_write_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def profiled_traffic(workload: str, B: int, P: int, algo: str, layout: str = "dense"):
    src_algo = "matrix" if algo.startswith("matrix") else algo
    """HBM bytes per attend dispatch from the committed rocprofv3 summary of
    this exact launch configuration
    (profiles/<kernel>_<workload>_b<B>_P<P>[_<layout>].md), scaled by the
    copy-kernel calibration recorded there; None if there is no such summary
    or the kernel source (with the device headers it includes) changed since
    it was taken."""
    f = _profile_fields(workload, B, P, algo, layout)
    if f.get("traffic_source_sha256_16") != source_hash((ATTEND_SOURCES[src_algo],) +
                                                        ATTEND_HEADERS):
        return None
    try:
        return int(f["read_bytes_per_dispatch"]) + int(f["write_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def interleave_cache(dev: dict, B: int, N: int, Hkv: int, D: int):
    """The cache as one row per cell: every head's K codes, then V codes,
    then K scales, then V scales (Hkv*(2D + D/8) bytes, each scale region
    padded to 16 bytes); returns device views
    at the four bases and the attention/append strides (bytes) that address
    them.  The four regions of a cell are disjoint, so the append writes and
    the attention reads the same cells as with the dense arrays.  (Padding
    the 1088-byte row to 1152 bytes, so every row starts on a 128-byte
    line, cut the decode attention's fetched bytes by 6% but made it 5%
    slower on this GPU; rows are not padded.)"""
    import torch
    codes, sc = Hkv * D, Hkv * (D // 32) * 2
    scp = (sc + 15) // 16 * 16         # each scale region 16-byte aligned
    row = 2 * codes + 2 * scp          # (1088 B for 2 heads of 256: no padding)
    buf = torch.zeros((B, N, row), dtype=torch.int8, device="cuda")
    buf[:, :, :codes].copy_(dev["Kq"].reshape(B, N, codes))
    buf[:, :, codes:2 * codes].copy_(dev["Vq"].reshape(B, N, codes))
    ks, vs = 2 * codes, 2 * codes + scp
    buf[:, :, ks:ks + sc].copy_(dev["Ksc"].reshape(B, N, -1).view(torch.int8))
    buf[:, :, vs:vs + sc].copy_(dev["Vsc"].reshape(B, N, -1).view(torch.int8))
    out = dict(dev)
    out["Kq"] = buf[:, :, :codes]
    out["Vq"] = buf[:, :, codes:2 * codes]
    out["Ksc"] = buf[:, :, ks:ks + sc]
    out["Vsc"] = buf[:, :, vs:vs + sc]
    out["kv_buffer"] = buf
    strides = {f"{n}_cell_stride": row for n in ("kq", "ksc", "vq", "vsc")}
    strides.update({f"{n}_batch_stride": row * N for n in ("kq", "ksc", "vq", "vsc")})
    return out, strides


def hbm_ceiling(inp: dict, dev: dict, path, B: int, P: int, attend_bytes: int,
                attend_ms: float) -> dict:
    """Attainable read rates measured by libhbm_probe.so on this GPU: one
    streaming read of 2 GiB, and (one-token workloads) the attention's cell
    gather alone -- the same kept ids, cache layout and split, no arithmetic.
    Rates are GB/s of bytes the kernels must read; the attention stage's own
    rate on its gathered bytes is given beside them."""
    import ctypes

    import torch

    from top_sparse_attention_score_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: run __graft_entry__.build()")
    L = ctypes.CDLL(PROBE_LIB)
    vp, ll, ci = ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int
    L.hbm_probe_stream.argtypes = [vp, ll, vp, ci, vp]
    L.hbm_probe_gather_sink_words.argtypes = [ci, ci, ci]
    L.hbm_probe_gather_sink_words.restype = ll
    L.hbm_probe_gather.argtypes = [vp] * 4 + [ll] * 8 + [vp] + [ci] * 5 + [vp, vp]
    stream = torch.cuda.current_stream()

    def timed(fn, n=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            rc = fn()
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    n = 2 << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    grid = 4096
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    t = timed(lambda: L.hbm_probe_stream(buf.data_ptr(), n, sink.data_ptr(), grid,
                                         stream.cuda_stream))
    del buf
    res = {"stream_read_gbs": round(n / t / 1e9, 1), "stream_bytes": n}
    if inp["T"] == 1 and int(path.n_sel.min().item()) == int(path.n_sel.max().item()):
        k = int(path.n_sel[0, 0].item())
        ids = path.ids[:, 0, :k].contiguous()
        a = path.adesc
        Hkv, D = inp["Hkv"], inp["D"]
        row, srow = Hkv * D, Hkv * (D // 32) * 2
        cs = [a.kq_cell_stride or row, a.vq_cell_stride or row, a.ksc_cell_stride or srow,
              a.vsc_cell_stride or srow]
        bs = [a.kq_batch_stride or cs[0] * inp["N"], a.vq_batch_stride or cs[1] * inp["N"],
              a.ksc_batch_stride or cs[2] * inp["N"], a.vsc_batch_stride or cs[3] * inp["N"]]
        gsink = torch.zeros(L.hbm_probe_gather_sink_words(B, Hkv, P), dtype=torch.int32,
                            device="cuda")
        t = timed(lambda: L.hbm_probe_gather(
            dev["Kq"].data_ptr(), dev["Vq"].data_ptr(), dev["Ksc"].data_ptr(),
            dev["Vsc"].data_ptr(), *cs, *bs, ids.data_ptr(), B, k, Hkv, D, P,
            gsink.data_ptr(), stream.cuda_stream))
        gathered = B * k * Hkv * (2 * D + D // 8)
        res.update(gather_gbs=round(gathered / t / 1e9, 1), gather_bytes=gathered,
                   gather_us=round(t * 1e6, 1),
                   attend_gather_gbs=round(gathered / (attend_ms * 1e-3) / 1e9, 1))
    return res


def warm_up_to_steady_clocks(step, stream, seconds: float = 0.1) -> None:
    """Untimed steps, enqueued back to back with no synchronisation between
    them, for about `seconds` of GPU time.  After a period of low load this
    GPU runs a sustained HBM-bound load about 7% slower for the first 10-30
    ms (measured: decode steps of ~250 us settling at ~236 us, and a warm-up
    broken by a host synchronisation every few milliseconds did not settle
    it), so the timed steps start only after one continuous run."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(10):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    per_step = max(e0.elapsed_time(e1) * 1e-3 / 10, 1e-6)
    for _ in range(int(math.ceil(seconds / per_step))):
        step()
    torch.cuda.synchronize()


def host_record() -> dict:
    """CPU model, logical CPUs and the CPUs this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return dict(cpu_model=model, nproc=os.cpu_count(), usable_cpus=usable)


def _oracle_problem(orc, inp_cfg: str, i: int, P: int) -> tuple[int, float]:
    """One sample problem of the workload through the oracle: (kept cells,
    seconds spent in the oracle call)."""
    from datagen import make_inputs
    inp = make_inputs(inp_cfg, seed=9000 + i, batch=1)
    if inp_cfg == "prompt":   # one token of the chunk per sample
        t = i % inp["T"]
        inp.update(T=1, pos0=inp["pos0"] + t, q_idx=inp["q_idx"][:, t:t + 1],
                   q=inp["q"][:, t:t + 1])
    t0 = time.perf_counter()
    r = orc.run(inp, P=P, scale=1.0 / math.sqrt(inp["D"]))
    return int(r["n_sel"].sum()), time.perf_counter() - t0


def cpu_baseline(inp_cfg: str, target_s: float, P: int) -> dict:
    """The oracle (plain C, double) on as many problems of the same workload
    as fit in about target_s seconds of oracle time on one thread (the
    reported value); then the same on every usable host CPU (up to 16), one
    thread each, for about half that time (reported beside it as the sum of
    the threads' rates).  Only the oracle calls are timed, not the input
    generation."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle.oracle import default
    orc = default()
    done, cells, t_used = 0, 0, 0.0
    while t_used < target_s:
        c, dt = _oracle_problem(orc, inp_cfg, done, P)
        cells += c
        t_used += dt
        done += 1
    what = "token" if inp_cfg == "prompt" else "problem"
    host = host_record()
    threads = max(1, min(16, host["usable_cpus"] or 1))

    def worker(w):
        n, c_w, t_w = 0, 0, 0.0
        while t_w < target_s / 2:
            c, dt = _oracle_problem(orc, inp_cfg, 10000 + 1000 * w + n, P)
            c_w, t_w, n = c_w + c, t_w + dt, n + 1
        return n, c_w / t_w

    with ThreadPoolExecutor(threads) as ex:
        per = list(ex.map(worker, range(threads)))
    return dict(value=cells / t_used, unit="cells/s", cores=1, kind="oracle",
                sample=f"{done} {what}(s) of the {inp_cfg} workload, index+attend+merge, "
                       f"{t_used:.1f} s of oracle time on one thread",
                host=host,
                all_cores=dict(value=sum(r for _, r in per), threads=threads,
                               sample=f"{sum(n for n, _ in per)} {what}(s) on {threads} "
                                      f"threads, ~{target_s / 2:.0f} s of oracle time each"))


def single_problem_latency(qsa, base: dict, P: int, algo_code: int, steps: int = 50) -> dict:
    """One problem (B = 1) per step, the latency-bound case: the same step
    (qsa_step: append -> index_topk -> attend -> gated merge) launched
    eagerly, and captured once in a HIP graph and replayed; then the step as
    the single cooperative launch of qsa_decode_window (eagerly and from a
    graph); microseconds per step."""
    import torch
    inp = {k: (v[:1] if hasattr(v, "shape") and getattr(v, "ndim", 0) and k in
               ("q_idx", "K_idx", "q", "Kq", "Ksc", "Vq", "Vsc") else v)
           for k, v in base.items()}
    inp["batch"] = 1
    dev = qsa.to_device(inp)
    gen = torch.Generator(device="cuda").manual_seed(99)
    T, Hkv, D, di = inp["T"], inp["Hkv"], inp["D"], inp["di"]
    k_new = torch.randn((1, T, Hkv, D), generator=gen, device="cuda")
    v_new = torch.randn((1, T, Hkv, D), generator=gen, device="cuda")
    i_new = torch.randn((1, T, di), generator=gen, device="cuda")
    dev["gate"] = torch.randn(tuple(dev["q"].shape), generator=gen,
                              device="cuda").to(dev["q"].dtype)
    adesc = qsa.append_desc(batch=1, T=T, n_cells=inp["N"], pos0=inp["pos0"], Hkv=Hkv, D=D,
                            d_idx=di)
    path = qsa.path_for(inp, P=P, algo=algo_code)
    side = torch.cuda.Stream()
    ws_step = torch.empty(qsa.qsa_step_workspace(path.idesc, path.adesc) // 4 + 64,
                          dtype=torch.int32, device="cuda")

    def step(stream=None):
        qsa.qsa_step(adesc, path.idesc, path.adesc, k_new, v_new, i_new, dev["Kq"], dev["Ksc"],
                     dev["Vq"], dev["Vsc"], dev["K_idx"], dev["q_idx"], dev["q"], dev["gate"],
                     path.ids, path.n_sel, path.out, ws_step, stream=stream)

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / steps * 1e3, 2)

    def graph_of(fn):
        g = torch.cuda.CUDAGraph()
        fn()
        torch.cuda.synchronize()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                fn(side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g

    res = dict(eager=timed(step), graph=timed(graph_of(step).replay))
    # The same step as one cooperative launch (qsa_decode_window), where the
    # library has a window kernel for the shape.
    ws_bytes = qsa.qsa_decode_window_workspace(path.idesc, path.adesc)
    if ws_bytes and T == 1 and not inp["q_dtype"] == "f16" and inp["pos0"] < 16384:
        ws = torch.empty(ws_bytes // 4 + 64, dtype=torch.int32, device="cuda")
        ids = torch.empty_like(path.ids)
        n_sel = torch.empty_like(path.n_sel)
        out = torch.empty_like(path.out)

        def window(stream=None):
            qsa.qsa_decode_window(adesc, path.idesc, path.adesc, k_new, v_new, i_new, dev["Kq"],
                                  dev["Ksc"], dev["Vq"], dev["Vsc"], dev["K_idx"],
                                  dev["q_idx"], dev["q"], dev["gate"], ids, n_sel, out, ws,
                                  stream=stream)
        res["window_eager"] = timed(window)
        res["window_graph"] = timed(graph_of(window).replay)
    return res


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--P", type=int, default=None)
    ap.add_argument("--distinct", type=int, default=8,
                    help="distinct seeded problems, tiled to the batch on the GPU")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-latency", action="store_true",
                    help="skip the single-problem (B = 1) latency measurement")
    ap.add_argument("--algo", default="matrix", choices=["matrix", "vector"],
                    help="qsa_attend kernel family")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the attainable-HBM-rate probes")
    ap.add_argument("--merge", default="fused", choices=["fused", "separate"],
                    help="attention and gated merge as one kernel (qsa_attend_merge, where "
                         "P is 1, 2 or 4) or as qsa_attend + qsa_merge_gated")
    ap.add_argument("--layout", default="interleaved", choices=["dense", "interleaved"],
                    help="KV cache layout: dense arrays [B][N][Hkv][D] and [B][N][Hkv][D/32], "
                         "or one row per cell holding every head's K codes, V codes, K "
                         "scales and V scales (strided views of one buffer)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB "
                         "(a known-size reference for rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import top_sparse_attention_score_amd as qsa
    from datagen import make_inputs

    cfg_name, default_batch, desc = WORKLOADS[args.workload]
    B = args.batch or default_batch
    nd = max(1, min(args.distinct, B))
    print(f"[bench] workload={args.workload} B={B} distinct={nd}", file=sys.stderr, flush=True)
    base = make_inputs(cfg_name, seed=1234, batch=nd)
    P = args.P or base["P"]
    reps = math.ceil(B / nd)
    dev = {}
    for key in ("q_idx", "K_idx", "q", "Kq", "Ksc", "Vq", "Vsc"):
        t = torch.from_numpy(base[key]).cuda()
        dev[key] = t.repeat((reps,) + (1,) * (t.dim() - 1))[:B].contiguous()
    inp = dict(base)
    inp["batch"] = B
    strides = None
    if args.layout == "interleaved":
        dev, strides = interleave_cache(dev, B, inp["N"], inp["Hkv"], inp["D"])
    algo_code = qsa.QSA_ATTEND_MATRIX if args.algo == "matrix" else qsa.QSA_ATTEND_VECTOR
    path = qsa.path_for(inp, P=P, algo=algo_code, strides=strides)
    # The step's new tokens (fp32 K / V / index rows, seeded) and their append.
    gen = torch.Generator(device="cuda").manual_seed(4321)
    T_new = inp["T"]
    k_new = torch.randn((B, T_new, inp["Hkv"], inp["D"]), generator=gen, device="cuda")
    v_new = torch.randn((B, T_new, inp["Hkv"], inp["D"]), generator=gen, device="cuda")
    i_new = torch.randn((B, T_new, inp["di"]), generator=gen, device="cuda")
    adesc = qsa.append_desc(batch=B, T=T_new, n_cells=inp["N"], pos0=inp["pos0"],
                            Hkv=inp["Hkv"], D=inp["D"], d_idx=inp["di"], strides=strides)
    gate = torch.randn(tuple(dev["q"].shape), generator=gen, device="cuda").to(dev["q"].dtype)
    dev["gate"] = gate

    def append():
        qsa.qsa_kv_append(adesc, k_new, v_new, i_new, dev["Kq"], dev["Ksc"], dev["Vq"],
                          dev["Vsc"], dev["K_idx"])

    fused = args.merge == "fused" and args.algo == "matrix" and P in (1, 2, 4)

    def attend_and_merge(ev=None):
        """attention + gated merge: one fused kernel, or the two calls (the
        event between them, if given, splits the two stages)."""
        if fused:
            path.attend_merge(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"],
                              gate=gate)
            if ev is not None:
                ev.record(stream)
        else:
            path.attend(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"])
            if ev is not None:
                ev.record(stream)
            path.merge(gate=gate)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 18        # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    # The step: one qsa_step call (append -> index -> attend -> gated merge
    # in the fewest launches the shape allows), marshalled once.
    ws_step = torch.empty(qsa.qsa_step_workspace(path.idesc, path.adesc) // 4 + 64,
                          dtype=torch.int32, device="cuda")
    step = qsa.StepCall(adesc, path.idesc, path.adesc, k_new, v_new, i_new, dev["Kq"],
                        dev["Ksc"], dev["Vq"], dev["Vsc"], dev["K_idx"], dev["q_idx"], dev["q"],
                        gate, path.ids, path.n_sel, path.out, ws_step, stream)
    if args.merge == "separate" or args.algo != "matrix":
        def step():  # noqa: F811  (the four calls, one by one)
            append()
            path.index(dev["q_idx"], dev["K_idx"])
            attend_and_merge()
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    n_sel_total = int(path.n_sel.sum().item())
    by = algorithmic_bytes(inp, B, n_sel_total)
    fused_att_bytes = by["attend"] + (by["out"] if fused else 0)

    def kernel_ms(fn, n=10):
        """Average duration of n back-to-back launches of one call on the
        launch stream (events around the n launches only)."""
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def attend_call():
        if fused:
            path.attend_merge(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"], gate=gate)
        else:
            path.attend(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"])

    # Attainable read rates of this GPU, measured before the timed steps (the
    # probes also bring the GPU to its working clocks).
    ceiling = None
    if not args.no_ceiling:
        ceiling = hbm_ceiling(inp, dev, path, B, P, fused_att_bytes,
                              kernel_ms(attend_call))
    # Last before the timed steps: one continuous run of untimed steps.
    warm_up_to_steady_clocks(step, stream, seconds=0.2)

    def timed_block():
        """K steps between two events on the launch stream (nothing else
        enqueued between them); microseconds per step."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(K):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    t_start = time.perf_counter()
    step_us0 = timed_block()                    # the reported K steps
    wall = time.perf_counter() - t_start
    rounds_us = np.array([step_us0] + [timed_block() for _ in range(4)])
    step_ms = step_us0 * 1e-3

    # Stage breakdown: each of the step's calls on its own, as the average of
    # ten back-to-back launches (every call is idempotent on these buffers:
    # the append rewrites the same cells with the same values).
    stage_ms = np.array([kernel_ms(append), kernel_ms(lambda: path.index(dev["q_idx"],
                                                                         dev["K_idx"])),
                         kernel_ms(attend_call),
                         0.0 if fused else kernel_ms(lambda: path.merge(gate=gate))])

    flops = attend_flops(inp, n_sel_total)
    cells_per_s = n_sel_total / (step_ms * 1e-3)
    gbs = by["total"] / (step_ms * 1e-3) / 1e9

    # Dominant kernel: the stage with the largest average time.  With the
    # fused kernel the attend stage includes the gated merge (its bytes: the
    # gate read and the output written) and the merge stage is empty.
    names = ["kv_append", "index_topk", "attend", "merge_gated"]
    if fused:
        names[2] = "attend_merge_gated"
    dom = int(np.argmax(stage_ms))
    att_bytes = fused_att_bytes
    # The attention kernel of this shape (its committed profile also holds
    # the index kernels' traffic): P a multiple of 4 above 4 with >= 512
    # (token, KV head) pairs runs several chunks per wave.
    mch = P % 4 == 0 and P > 4 and B * inp["T"] * inp["Hkv"] >= 512
    kalgo = ("matrix_merge" if fused else ("matrix_mch" if mch else "matrix")) \
        if args.algo == "matrix" else args.algo
    att_ms = stage_ms[2]
    if names[dom] == "attend" and args.algo == "vector":
        achieved = flops / (att_ms * 1e-3) / 1e12
        roof = dict(kernel="k_attend", bound="alu", achieved=round(achieved, 2),
                    peak=round(FP32_VALU_PEAK_TFLOPS, 1), unit="TFLOP/s",
                    frac=round(achieved / FP32_VALU_PEAK_TFLOPS, 4),
                    traffic=profiled_traffic(args.workload, B, P, args.algo, args.layout),
                    algorithmic_bytes=by["attend"],
                    hbm_gbs=round(by["attend"] / (att_ms * 1e-3) / 1e9, 1))
    elif dom == 2:
        # Matrix kernel: the products run on the matrix cores far below
        # their peak; the gathers of the kept cells bound it.
        achieved = att_bytes / (att_ms * 1e-3) / 1e9
        roof = dict(kernel=ATTEND_KERNELS[kalgo], bound="hbm", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=profiled_traffic(args.workload, B, P, kalgo, args.layout),
                    algorithmic_bytes=att_bytes,
                    definition_tflops=round(flops / (att_ms * 1e-3) / 1e12, 2))
    else:
        sb = {"index_topk": by["index"], "merge_gated": by["out"],
              "kv_append": by["append"]}[names[dom]]
        achieved = sb / (stage_ms[dom] * 1e-3) / 1e9
        traffic = (profiled_index_traffic(args.workload, B, P, kalgo, args.layout)
                   if names[dom] == "index_topk" else None)
        roof = dict(kernel=names[dom], bound="hbm", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=traffic, algorithmic_bytes=sb)

    line = {
        "metric": METRIC, "value": cells_per_s, "unit": "cells/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": desc, "batch": B, "T": inp["T"], "n_cells": inp["N"],
                   "k": inp["k"], "P": P, "d_idx": inp["di"], "heads": f"{inp['Hq']}x{inp['D']}",
                   "kv_heads": inp["Hkv"], "attend_kernel": args.algo,
                   "merge": "fused" if fused else "separate",
                   "kv_layout": args.layout},
        "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": by["total"],
        "stage_us": {n: round(float(v) * 1e3, 2) for n, v in zip(names, stage_ms)
                     if not (fused and n == "merge_gated")},
        "step_us": {"timed": round(step_us0, 2), "rounds": len(rounds_us),
                    "median": round(float(np.median(rounds_us)), 2),
                    "min": round(float(rounds_us.min()), 2),
                    "max": round(float(rounds_us.max()), 2)},
        "launch": "qsa_step" if step.__class__.__name__ == "StepCall" else "separate calls",
        "wall_s": round(wall, 3),
        "roofline": roof,
    }
    if inp["q_dtype"] == "f16":
        line["dtype"] = "f16 in, f32 accumulate"
    if ceiling is not None:
        line["hbm_ceiling"] = ceiling
    if not args.no_latency:
        p_lat = LATENCY_P.get(args.workload, P)
        line["latency_b1_us"] = dict(P=p_lat, **single_problem_latency(qsa, base, p_lat, algo_code))
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg_name, args.cpu_seconds, P)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
