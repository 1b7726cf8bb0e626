"""The oracle over many tokens on the host's cores.

The C oracle runs one call per slice of consecutive tokens; ctypes releases
the GIL during each call, so slices run in parallel threads.  Each slice is
the same computation as one call over all tokens (tokens are independent:
token t sees cells 0..pos0+t whatever the slice), so the result does not
depend on the slicing.
"""
from __future__ import annotations

import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from tests.gpu_util import say


def host_threads(cap: int = 16) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def oracle_all_tokens(orc, inp: dict, *, P: int, scale: float, slice_tokens: int = 8,
                      threads: int | None = None) -> dict:
    """ids, n_sel and out of every token of every problem of `inp`, computed
    by the oracle in slices of `slice_tokens` tokens on `threads` threads."""
    B, T = inp["q"].shape[:2]
    cap = inp["cap"]
    ids = np.empty((B, T, cap), np.int32)
    n_sel = np.empty((B, T), np.int32)
    out = np.empty(inp["q"].shape, np.float64)
    jobs = [(b, t0, min(T, t0 + slice_tokens)) for b in range(B)
            for t0 in range(0, T, slice_tokens)]
    done = [0]
    lock = threading.Lock()

    def one(job):
        b, t0, t1 = job
        sub = dict(inp)
        sub.update(T=t1 - t0, pos0=inp["pos0"] + t0, batch=1,
                   q_idx=inp["q_idx"][b:b + 1, t0:t1], q=inp["q"][b:b + 1, t0:t1],
                   K_idx=inp["K_idx"][b:b + 1], Kq=inp["Kq"][b:b + 1],
                   Ksc=inp["Ksc"][b:b + 1], Vq=inp["Vq"][b:b + 1], Vsc=inp["Vsc"][b:b + 1])
        r = orc.run(sub, P=P, scale=scale)
        ids[b, t0:t1], n_sel[b, t0:t1], out[b, t0:t1] = r["ids"][0], r["n_sel"][0], r["out"][0]
        with lock:
            done[0] += 1
            if done[0] % 32 == 0 or done[0] == len(jobs):
                say(f"[oracle pool] {done[0]}/{len(jobs)} slices")

    with ThreadPoolExecutor(threads or host_threads()) as ex:
        list(ex.map(one, jobs))
    return dict(ids=ids, n_sel=n_sel, out=out)
