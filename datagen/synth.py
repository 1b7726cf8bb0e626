"""Seeded synthetic inputs for the QSA path.

The audit pages test their kernels on random data (random int8 KV with fp16
scales, top-k-shaped or randomly scattered ids, a 32768-cell cache swept over
pos0 in {0,1,63,64,512,2047,2048,2050,8192,30000} x ntok in {1,2,4,8}); no
public dataset is involved.  These generators produce inputs of the same
shapes and kinds:

* index queries and keys: N(0,1) rounded to the 2^-5 grid and clamped to
  [-4, 4], stored as fp16 (every such value is exact in fp16).  With
  ``index_grid=False`` they are N(0,1) rounded to the nearest fp16 instead
  (general fp16 keys, where fp32 score sums depend on the summation order).
  On the grid
  every fp16 x fp16 product is a multiple of 2^-10 of magnitude <= 16, so every
  partial sum of up to 1024 such products is a multiple of 2^-10 below 2^14 and
  is exact in fp32 (24-bit significand): scores computed in fp32 in any
  order equal the double-precision scores bit for bit, which is what makes the
  top-k ids comparable bit-exactly.
* KV cache: int8 codes clip(round(36 z), -127, 127) with z ~ N(0,1), and one
  fp16 scale per 32 elements of a (cell, KV head) row drawn as U(0.75,1.25)/36,
  so dequantised values are roughly N(0,1).  No quantiser is involved: the
  codes and scales are the random inputs.
* queries: N(0,1), fp32 (fp16 for the prompt-chunk workload).
* long-context workload: 5% of cells (Bernoulli mask) get index key
  r + 3 q_hat (q_hat the unit index query), which gives them scores around
  +3 sigma (a planted heavy tail); 1% of planted cells then copy another
  planted cell's key row, forcing exactly equal scores.

Layouts match the library's dense layouts (see include/qsa.h):
  q_idx [B][T][di]  K_idx [B][N][di]  q [B][T][Hq][D]
  Kq, Vq [B][N][Hkv][D] int8   Ksc, Vsc [B][N][Hkv][D/32] fp16
"""
from __future__ import annotations

import numpy as np

# Workloads.  T query tokens sit at positions pos0..pos0+T-1 with
# pos0 = N - T (the last T cells) unless overridden.
CONFIGS = {
    # 1 token, 4 q heads x 64, 1 KV head, 512 cells, index dim 64, top-128,
    # 4 split-KV partials.
    "tiny": dict(T=1, N=512, di=64, k=128, dense_max=131, Hq=4, Hkv=1, D=64, P=4,
                 q_dtype="f32", out_dtype="f32", heavy_tail=False),
    # 1 token, 24 q heads x 256, 2 KV heads, 8192 cells, index dim 128, top-2048,
    # 4 split-KV partials (chunks of 512 kept cells).
    "decode": dict(T=1, N=8192, di=128, k=2048, dense_max=2051, Hq=24, Hkv=2, D=256,
                   P=4, q_dtype="f32", out_dtype="f32", heavy_tail=False),
    # 8 draft tokens, 65536 cells, 16 partials per token.
    "draft": dict(T=8, N=65536, di=128, k=2048, dense_max=2051, Hq=24, Hkv=2, D=256,
                  P=16, q_dtype="f32", out_dtype="f32", heavy_tail=False),
    # 1 token, 262144 cells, planted heavy tail, 64 partials.
    "long": dict(T=1, N=262144, di=128, k=2048, dense_max=2051, Hq=24, Hkv=2, D=256,
                 P=64, q_dtype="f32", out_dtype="f32", heavy_tail=True),
    # 2048-token prompt chunk against 65536 cells, fp16 q and output.
    "prompt": dict(T=2048, N=65536, di=128, k=2048, dense_max=2051, Hq=24, Hkv=2,
                   D=256, P=1, q_dtype="f16", out_dtype="f16", heavy_tail=False),
}

# The pos0 x ntok sweep of the pages' bitwise check, on a 32768-cell cache.
SWEEP_POS0 = (0, 1, 63, 64, 512, 2047, 2048, 2050, 8192, 30000)
SWEEP_NTOK = (1, 2, 4, 8)


def sweep_cases():
    for pos0 in SWEEP_POS0:
        for ntok in SWEEP_NTOK:
            yield pos0, ntok


def _grid16(x: np.ndarray) -> np.ndarray:
    """Round to the 2^-5 grid, clamp to [-4, 4], store as fp16 (exact)."""
    return np.clip(np.round(x * 32.0) / 32.0, -4.0, 4.0).astype(np.float16)


def _raw16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest fp16 (no grid)."""
    return x.astype(np.float16)


def _kv(rng: np.random.Generator, B: int, N: int, Hkv: int, D: int):
    z = rng.standard_normal((B, N, Hkv, D), dtype=np.float32)
    codes = np.clip(np.rint(z * 36.0), -127, 127).astype(np.int8)
    u = rng.uniform(0.75, 1.25, size=(B, N, Hkv, D // 32))
    scales = (u / 36.0).astype(np.float16)
    return codes, scales


def make_inputs(cfg="decode", *, seed: int = 1000, batch: int = 1, **over) -> dict:
    """Seeded inputs for one workload.  ``cfg`` is a CONFIGS key or a dict;
    keyword overrides replace any parameter (e.g. N, T, pos0, k, P)."""
    p = dict(CONFIGS[cfg]) if isinstance(cfg, str) else dict(cfg)
    p.update(over)
    T, N, di, Hq, Hkv, D = p["T"], p["N"], p["di"], p["Hq"], p["Hkv"], p["D"]
    p.setdefault("pos0", N - T)
    p.setdefault("cap", max(p["k"], p["dense_max"]))
    B = batch
    rng = np.random.default_rng(seed)
    to16 = _grid16 if p.get("index_grid", True) else _raw16

    q_idx_f = rng.standard_normal((B, T, di))
    q_idx = to16(q_idx_f)
    K_raw = rng.standard_normal((B, N, di))
    if p.get("heavy_tail"):
        for b in range(B):
            qv = q_idx[b, 0].astype(np.float64)
            q_hat = qv / max(np.linalg.norm(qv), 1e-30)
            mask = rng.random(N) < 0.05
            K_raw[b, mask] += 3.0 * q_hat
            K_b = to16(K_raw[b])
            planted = np.flatnonzero(mask)
            if planted.size >= 2:
                n_copy = max(1, planted.size // 100)
                dst = rng.choice(planted, size=n_copy, replace=False)
                src = rng.choice(planted, size=n_copy, replace=True)
                K_b[dst] = K_b[src]
            K_raw[b] = K_b.astype(np.float64)
    K_idx = to16(K_raw)

    if p["q_dtype"] == "f16":
        q = rng.standard_normal((B, T, Hq, D), dtype=np.float32).astype(np.float16)
    else:
        q = rng.standard_normal((B, T, Hq, D), dtype=np.float32)
    Kq, Ksc = _kv(rng, B, N, Hkv, D)
    Vq, Vsc = _kv(rng, B, N, Hkv, D)
    out = dict(p)
    out.update(q_idx=q_idx, K_idx=K_idx, q=q, Kq=Kq, Ksc=Ksc, Vq=Vq, Vsc=Vsc,
               batch=B, seed=seed)
    return out


def scattered_ids(*, seed: int, batch: int, T: int, N: int, cap: int, pos0: int,
                  n_max: int) -> tuple[np.ndarray, np.ndarray]:
    """Random scattered id rows (the pages' attention-only test input):
    token t keeps min(n_max, pos0+t+1) distinct visible cells, ascending,
    rows padded with -1."""
    rng = np.random.default_rng(seed)
    ids = np.full((batch, T, cap), -1, dtype=np.int32)
    n_sel = np.zeros((batch, T), dtype=np.int32)
    for b in range(batch):
        for t in range(T):
            nvis = pos0 + t + 1
            n = min(n_max, nvis, cap)
            sel = np.sort(rng.choice(nvis, size=n, replace=False)).astype(np.int32)
            ids[b, t, :n] = sel
            n_sel[b, t] = n
    return ids, n_sel
