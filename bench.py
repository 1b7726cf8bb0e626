"""Throughput benchmark of the QSA hot path on one MI355X.

One step = qsa_kv_append -> qsa_index_topk -> qsa_attend -> qsa_merge_gated
over a batch of B independent problems (seeded synthetic caches already
resident in HBM): the step's T new tokens are quantised into their cells of
the cache, then selected from and attended to, and the merged output is
gated.
The default workload is the decode step (1 token, 24 x 256 query heads,
2 KV heads, 8192 cached cells, index dim 128, top-2048) over B = 256
independent caches, so the working set (~2.7 GB) is far larger than the
256 MB last-level cache and every step streams from HBM.

Prints one JSON line: metric/value (kept KV cells attended per second),
per-stage times from HIP events recorded on the launch stream, algorithmic
HBM bytes and flops, the roofline of the dominant kernel, and the oracle's
single-thread throughput on a bounded sample of the same workload.
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
    "decode": ("decode", 256, "decode step: 1 token, 24x256 q heads, 2 KV heads, 8192 cells, "
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
ATTEND_KERNELS = {"matrix": "k_attend_mma", "vector": "k_attend"}
# Headers whose code the attend kernels compile in (also hashed).
ATTEND_HEADERS = ("qsa_device.h", "qsa_mma.h")


def profiled_traffic(workload: str, B: int, P: int, algo: str):
    """HBM bytes per attend dispatch from the committed rocprofv3 summary of
    this exact launch configuration (profiles/<kernel>_<workload>_b<B>_P<P>.md),
    scaled by the copy-kernel calibration recorded there; None if there is no
    such summary or the kernel source (with the device headers it includes)
    changed since it was taken."""
    import hashlib
    kern = ATTEND_KERNELS[algo]
    path = os.path.join(ROOT, "profiles", f"{kern}_{workload}_b{B}_P{P}.md")
    src = os.path.join(ROOT, "top_sparse_attention_score_amd", "csrc", ATTEND_SOURCES[algo])
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    sha = hashlib.sha256(b"".join(open(f, "rb").read() for f in [src] + [
        os.path.join(os.path.dirname(src), h) for h in ATTEND_HEADERS])).hexdigest()[:16]
    if fields.get("traffic_source_sha256_16") != sha:
        return None
    try:
        return int(fields["read_bytes_per_dispatch"]) + int(fields["write_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp_cfg: str, target_s: float, P: int) -> dict:
    """The oracle (plain C, double, one thread) on as many problems of the same
    workload as fit in about target_s seconds."""
    from datagen import make_inputs
    from oracle.oracle import default
    orc = default()
    done, cells, t_used = 0, 0, 0.0
    seed = 9000
    while t_used < target_s:
        inp = make_inputs(inp_cfg, seed=seed + done, batch=1)
        if inp_cfg == "prompt":   # one token of the chunk per sample
            t = done % inp["T"]
            inp.update(T=1, pos0=inp["pos0"] + t, q_idx=inp["q_idx"][:, t:t + 1],
                       q=inp["q"][:, t:t + 1])
        t0 = time.perf_counter()
        r = orc.run(inp, P=P, scale=1.0 / math.sqrt(inp["D"]))
        t_used += time.perf_counter() - t0
        cells += int(r["n_sel"].sum())
        done += 1
    unit = "cells/s"
    what = "token" if inp_cfg == "prompt" else "problem"
    return dict(value=cells / t_used, unit=unit, cores=1, kind="oracle",
                sample=f"{done} {what}(s) of the {inp_cfg} workload, index+attend+merge, "
                       f"{t_used:.1f} s single-threaded")


def single_problem_latency(qsa, base: dict, P: int, algo_code: int, steps: int = 50) -> dict:
    """One problem (B = 1) per step, the latency-bound case: the same step
    (append -> index_topk -> attend -> gated merge) launched eagerly, and
    captured once in a HIP graph and replayed; microseconds per step."""
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

    def step(stream=None):
        qsa.qsa_kv_append(adesc, k_new, v_new, i_new, dev["Kq"], dev["Ksc"], dev["Vq"],
                          dev["Vsc"], dev["K_idx"], stream=stream)
        path.run(dev, stream=stream)

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

    eager = timed(step)
    g = torch.cuda.CUDAGraph()
    step()
    torch.cuda.synchronize()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return dict(eager=eager, graph=timed(g.replay))


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
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
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB "
                         "(a known-size reference for rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path", file=sys.stderr)
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
    algo_code = qsa.QSA_ATTEND_MATRIX if args.algo == "matrix" else qsa.QSA_ATTEND_VECTOR
    path = qsa.path_for(inp, P=P, algo=algo_code)
    # The step's new tokens (fp32 K / V / index rows, seeded) and their append.
    gen = torch.Generator(device="cuda").manual_seed(4321)
    T_new = inp["T"]
    k_new = torch.randn((B, T_new, inp["Hkv"], inp["D"]), generator=gen, device="cuda")
    v_new = torch.randn((B, T_new, inp["Hkv"], inp["D"]), generator=gen, device="cuda")
    i_new = torch.randn((B, T_new, inp["di"]), generator=gen, device="cuda")
    adesc = qsa.append_desc(batch=B, T=T_new, n_cells=inp["N"], pos0=inp["pos0"],
                            Hkv=inp["Hkv"], D=inp["D"], d_idx=inp["di"])
    gate = torch.randn(tuple(dev["q"].shape), generator=gen, device="cuda").to(dev["q"].dtype)
    dev["gate"] = gate

    def append():
        qsa.qsa_kv_append(adesc, k_new, v_new, i_new, dev["Kq"], dev["Ksc"], dev["Vq"],
                          dev["Vsc"], dev["K_idx"])
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
    for _ in range(W):
        append()
        path.run(dev)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    t_start = time.perf_counter()
    for s in range(K):
        e = evs[s]
        e[0].record(stream)
        append()
        e[1].record(stream)
        path.index(dev["q_idx"], dev["K_idx"])
        e[2].record(stream)
        path.attend(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"])
        e[3].record(stream)
        path.merge(gate=gate)
        e[4].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    stage = np.zeros(4)
    for e in evs:
        for i in range(4):
            stage[i] += e[i].elapsed_time(e[i + 1])
    stage_ms = stage / K
    step_ms = float(evs[0][0].elapsed_time(evs[-1][4])) / K

    n_sel_total = int(path.n_sel.sum().item())
    by = algorithmic_bytes(inp, B, n_sel_total)
    flops = attend_flops(inp, n_sel_total)
    cells_per_s = n_sel_total / (step_ms * 1e-3)
    gbs = by["total"] / (step_ms * 1e-3) / 1e9

    # Dominant kernel: the stage with the largest average time.
    names = ["kv_append", "index_topk", "attend", "merge_gated"]
    dom = int(np.argmax(stage_ms))
    att_ms = stage_ms[2]
    if names[dom] == "attend" and args.algo == "vector":
        achieved = flops / (att_ms * 1e-3) / 1e12
        roof = dict(kernel="k_attend", bound="alu", achieved=round(achieved, 2),
                    peak=round(FP32_VALU_PEAK_TFLOPS, 1), unit="TFLOP/s",
                    frac=round(achieved / FP32_VALU_PEAK_TFLOPS, 4),
                    traffic=profiled_traffic(args.workload, B, P, args.algo),
                    algorithmic_bytes=by["attend"],
                    hbm_gbs=round(by["attend"] / (att_ms * 1e-3) / 1e9, 1))
    elif names[dom] == "attend":
        # Matrix kernel: the products run on the matrix cores far below
        # their peak; the gathers of the kept cells bound it.
        achieved = by["attend"] / (att_ms * 1e-3) / 1e9
        roof = dict(kernel="k_attend_mma", bound="hbm", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=profiled_traffic(args.workload, B, P, args.algo),
                    algorithmic_bytes=by["attend"],
                    definition_tflops=round(flops / (att_ms * 1e-3) / 1e12, 2))
    else:
        sb = {"index_topk": by["index"], "merge_gated": by["out"],
              "kv_append": by["append"]}[names[dom]]
        achieved = sb / (stage_ms[dom] * 1e-3) / 1e9
        roof = dict(kernel=names[dom], bound="hbm", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=None)

    line = {
        "metric": METRIC, "value": cells_per_s, "unit": "cells/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": desc, "batch": B, "T": inp["T"], "n_cells": inp["N"],
                   "k": inp["k"], "P": P, "d_idx": inp["di"], "heads": f"{inp['Hq']}x{inp['D']}",
                   "kv_heads": inp["Hkv"], "attend_kernel": args.algo},
        "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": by["total"],
        "stage_us": {n: round(float(v) * 1e3, 2) for n, v in zip(names, stage_ms)},
        "wall_s": round(wall, 3),
        "roofline": roof,
    }
    if inp["q_dtype"] == "f16":
        line["dtype"] = "f16 in, f32 accumulate"
    if not args.no_latency:
        p_lat = LATENCY_P.get(args.workload, P)
        line["latency_b1_us"] = dict(P=p_lat, **single_problem_latency(qsa, base, p_lat, algo_code))
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg_name, args.cpu_seconds, P)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
