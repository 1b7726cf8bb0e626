"""Pins of the double-precision oracle to things other than itself.

Each ``pin_*`` function takes a loaded oracle build and raises AssertionError
when it disagrees with what the pages and the mathematics fix:

* library routines on cases that reduce to them: numpy's IEEE binary16
  conversions, numpy float64 matrix products for the index scores,
  ``np.lexsort`` for the ranked selection, ``scipy.special.softmax`` for
  dense attention over the kept cells;
* closed forms: a token at position 0 attends to cell 0 only, so its output
  is that cell's dequantised V row exactly; q = 0 gives the mean V row;
  identical V rows give that row;
* invariants: re-associating the softmax into any number of chunks leaves the
  merged output unchanged; k >= visible cells equals dense attention;
  the kept set dominates the rest in score, ties going to lower indices;
* hand-derived worked examples stored under tests/golden/;
* the KV quantiser against exact rational arithmetic (Python fractions over
  numpy's binary16 table), including constructed ties and subnormal scales.

The same functions are run against deliberately broken copies of the oracle
(tests/test_oracle_mutants.py) to show that each plausible mistake fails at
least one of them.
"""
from __future__ import annotations

import bisect
import glob
import json
import math
import os
from fractions import Fraction

import numpy as np
from scipy.special import softmax

from datagen import make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def _deq(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """int8 codes x fp16 scale of each 32-element block, in float64."""
    return codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 32, axis=-1)


def _cfg(**kw):
    base = dict(T=1, N=64, di=8, k=8, dense_max=4, Hq=2, Hkv=1, D=32, P=2,
                q_dtype="f32", out_dtype="f32", heavy_tail=False)
    base.update(kw)
    return base


def _dense_reference(inp, ids, n_sel, scale):
    """Brute-force attention over each token's kept cells with scipy softmax."""
    q = inp["q"].astype(np.float64)
    Kh, Vh = _deq(inp["Kq"], inp["Ksc"]), _deq(inp["Vq"], inp["Vsc"])
    B, T, Hq, D = q.shape
    G = Hq // inp["Hkv"]
    out = np.zeros((B, T, Hq, D))
    for b in range(B):
        for t in range(T):
            sel = ids[b, t, : n_sel[b, t]]
            for h in range(Hq):
                g = h // G
                x = scale * (Kh[b, sel, g, :] @ q[b, t, h])
                out[b, t, h] = softmax(x) @ Vh[b, sel, g, :]
    return out


# ------------------------------------------------------------------ fp16 ---

def pin_half_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = orc.half_to_double(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero is kept
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_half_encode(orc):
    rng = np.random.default_rng(11)
    finite = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = np.sort(finite[np.isfinite(finite)].astype(np.float64))
    finite = np.unique(finite)
    # exact midpoints between neighbouring binary16 values (ties to even)
    mids = (finite[:-1] + finite[1:]) / 2.0
    sel = rng.choice(mids.size, size=3000, replace=False)
    xs = [mids[sel], finite[rng.choice(finite.size, 2000, replace=False)],
          rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 6, size=3000),
          np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 7e4, -7e4, 2.0 ** -24,
                    2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 6.1e-5,
                    np.inf, -np.inf, 1e300, -1e300])]
    x = np.concatenate(xs)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = orc.double_to_half(x)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:5]


# ------------------------------------------------------------ index/topk ---

def pin_scores_matmul(orc):
    """Scores equal a float64 matrix product of the fp16 inputs (exactly on
    the 2^-5 grid, to rounding on raw fp16 values)."""
    inp = make_inputs(_cfg(T=3, N=300, di=64, k=16, dense_max=8), seed=3)
    _, _, sc = orc.index_topk(inp["q_idx"], inp["K_idx"], k=16, pos0=inp["pos0"],
                              dense_max=8, cap=16, want_scores=True)
    S = inp["q_idx"][0].astype(np.float64) @ inp["K_idx"][0].astype(np.float64).T
    for t in range(3):
        nvis = inp["pos0"] + t + 1
        assert np.array_equal(sc[0, t, :nvis], S[t, :nvis])
        assert np.isnan(sc[0, t, nvis:]).all()
    rng = np.random.default_rng(5)
    qr = rng.standard_normal((1, 2, 128)).astype(np.float16)
    kr = rng.standard_normal((1, 200, 128)).astype(np.float16)
    _, _, sc = orc.index_topk(qr, kr, k=4, pos0=198, dense_max=0, cap=4,
                              want_scores=True)
    S = qr[0].astype(np.float64) @ kr[0].astype(np.float64).T
    assert np.allclose(sc[0, 0, :199], S[0, :199], rtol=1e-12, atol=1e-12)
    assert np.allclose(sc[0, 1], S[1], rtol=1e-12, atol=1e-12)
    assert np.isnan(sc[0, 0, 199])


def _expected_selection(S_row, nvis, k, dense_max):
    if nvis <= dense_max:
        return np.arange(nvis)
    order = np.lexsort((np.arange(nvis), -S_row[:nvis]))
    return np.sort(order[:k])


def pin_topk_bruteforce(orc):
    """Ranked selection against np.lexsort on small cases full of exact ties."""
    rng = np.random.default_rng(7)
    for _ in range(60):
        T = int(rng.integers(1, 5))
        N = int(rng.integers(T, 300))
        di = int(rng.choice([1, 2, 3, 8]))
        q_idx = rng.integers(-2, 3, size=(1, T, di)).astype(np.float16)
        K_idx = rng.integers(-2, 3, size=(1, N, di)).astype(np.float16)
        k = int(rng.integers(1, 40))
        dense_max = int(rng.integers(0, 60))
        cap = max(k, dense_max) + int(rng.integers(0, 3))
        pos0 = int(rng.integers(0, N - T + 1))
        ids, n_sel = orc.index_topk(q_idx, K_idx, k=k, pos0=pos0,
                                    dense_max=dense_max, cap=cap)
        S = q_idx[0].astype(np.float64) @ K_idx[0].astype(np.float64).T
        for t in range(T):
            nvis = pos0 + t + 1
            exp = _expected_selection(S[t], nvis, k, dense_max)
            n = len(exp)
            assert n_sel[0, t] == n
            assert np.array_equal(ids[0, t, :n], exp)
            assert (ids[0, t, n:] == -1).all()


def pin_dense_boundary(orc):
    """The dense fallback applies exactly while visible cells <= dense_max."""
    rng = np.random.default_rng(17)
    N, di, k, dm = 64, 4, 5, 9
    q_idx = rng.integers(-3, 4, size=(1, 1, di)).astype(np.float16)
    K_idx = rng.integers(-3, 4, size=(1, N, di)).astype(np.float16)
    for pos0 in (0, dm - 2, dm - 1, dm, dm + 1, N - 1):
        ids, n_sel = orc.index_topk(q_idx, K_idx, k=k, pos0=pos0, dense_max=dm, cap=dm)
        nvis = pos0 + 1
        if nvis <= dm:
            assert n_sel[0, 0] == nvis
            assert np.array_equal(ids[0, 0, :nvis], np.arange(nvis))
        else:
            assert n_sel[0, 0] == k


def pin_topk_invariants(orc):
    """On the heavy-tail workload: every kept score >= every dropped visible
    score, ties at the threshold go to lower indices, k ids ascending."""
    inp = make_inputs("long", seed=21, N=20000, k=512, dense_max=515)
    ids, n_sel, sc = orc.index_topk(inp["q_idx"], inp["K_idx"], k=512,
                                    pos0=inp["pos0"], dense_max=515, cap=515,
                                    want_scores=True)
    n = n_sel[0, 0]
    assert n == 512
    kept = ids[0, 0, :n]
    assert np.all(np.diff(kept) > 0)
    s = sc[0, 0, : inp["pos0"] + 1]
    mask = np.zeros(s.size, bool)
    mask[kept] = True
    lo = s[mask].min()
    assert s[~mask].max() <= lo
    tied_out = np.flatnonzero((~mask) & (s == lo))
    tied_in = np.flatnonzero(mask & (s == lo))
    if tied_out.size:
        assert tied_in.max() < tied_out.min()


# --------------------------------------------------------------- attend ---

def pin_attention_bruteforce(orc):
    """Chunked partials + merge == scipy softmax over the kept cells."""
    rng = np.random.default_rng(23)
    for trial in range(14):
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 3, 4]))
        D = int(rng.choice([32, 64]))
        T = int(rng.integers(1, 4))
        N = int(rng.integers(40, 160))
        k = int(rng.integers(3, 30))
        P = int(rng.integers(1, 7))
        qd = "f16" if trial % 3 == 0 else "f32"
        inp = make_inputs(_cfg(T=T, N=N, di=8, k=k, dense_max=k + 3, Hq=Hkv * G,
                               Hkv=Hkv, D=D, P=P, q_dtype=qd), seed=100 + trial,
                          pos0=int(rng.integers(0, N - T + 1)))
        scale = float(rng.choice([1.0 / math.sqrt(D), 0.3]))
        res = orc.run(inp, P=P, scale=scale)
        ref = _dense_reference(inp, res["ids"], res["n_sel"], scale)
        assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-14)


def pin_closed_forms(orc):
    # (i) position 0: one visible cell -> output is its dequantised V row.
    inp = make_inputs(_cfg(T=1, N=16, Hq=4, Hkv=2, D=64, P=3), seed=31, pos0=0)
    res = orc.run(inp, P=3)
    Vh = _deq(inp["Vq"], inp["Vsc"])
    assert res["n_sel"][0, 0] == 1 and res["ids"][0, 0, 0] == 0
    for h in range(4):
        assert np.array_equal(res["out"][0, 0, h], Vh[0, 0, h // 2])
    # (ii) q = 0: uniform weights -> mean of the kept V rows.
    inp = make_inputs(_cfg(T=2, N=90, k=20, dense_max=23, Hq=2, Hkv=2, D=32, P=4),
                      seed=32)
    inp["q"][:] = 0
    res = orc.run(inp, P=4)
    Vh = _deq(inp["Vq"], inp["Vsc"])
    for t in range(2):
        sel = res["ids"][0, t, : res["n_sel"][0, t]]
        for h in range(2):
            assert np.allclose(res["out"][0, t, h], Vh[0, sel, h].mean(axis=0),
                               rtol=1e-13, atol=1e-15)
    # (iii) identical V rows: any weights give that row.
    inp = make_inputs(_cfg(T=1, N=70, k=12, dense_max=15, Hq=3, Hkv=1, D=32, P=5),
                      seed=33)
    inp["Vq"][:] = inp["Vq"][:, :1]
    inp["Vsc"][:] = inp["Vsc"][:, :1]
    res = orc.run(inp, P=5)
    Vh = _deq(inp["Vq"], inp["Vsc"])
    for h in range(3):
        assert np.allclose(res["out"][0, 0, h], Vh[0, 0, 0], rtol=1e-13, atol=1e-15)


def pin_k_covers_all(orc):
    """k >= visible cells: top-k keeps every visible cell and the output is
    dense causal attention."""
    inp = make_inputs(_cfg(T=3, N=50, k=64, dense_max=2, Hq=2, Hkv=1, D=32, P=3),
                      seed=41, pos0=30)
    res = orc.run(inp, P=3)
    for t in range(3):
        nvis = 30 + t + 1
        assert res["n_sel"][0, t] == nvis
        assert np.array_equal(res["ids"][0, t, :nvis], np.arange(nvis))
    ref = _dense_reference(inp, res["ids"], res["n_sel"], 1.0 / math.sqrt(32))
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-14)


def pin_split_invariance(orc):
    """Re-associating the softmax into P chunks (including empty ones) does
    not change the merged output."""
    inp = make_inputs(_cfg(T=2, N=200, k=37, dense_max=40, Hq=4, Hkv=2, D=64, P=1),
                      seed=51)
    ids, n_sel = orc.index_topk(inp["q_idx"], inp["K_idx"], k=37, pos0=inp["pos0"],
                                dense_max=40, cap=40)
    outs = []
    for P in (1, 2, 3, 4, 16, 32, 37, 64):
        pm, pl, po = orc.attend(inp["q"], inp["Kq"], inp["Ksc"], inp["Vq"], inp["Vsc"],
                                ids, n_sel, P=P, scale=0.125)
        outs.append(orc.merge(pm, pl, po))
        if P > 37:   # more chunks than ids: trailing chunks are empty
            assert np.all(pm[..., 37:] == -np.inf) and np.all(pl[..., 37:] == 0)
            assert np.all(po[..., 37:, :] == 0)
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=1e-12, atol=1e-15)


def pin_merge_textbook(orc):
    """Merging chunk partials equals the textbook softmax over all logits."""
    rng = np.random.default_rng(61)
    for _ in range(20):
        n = int(rng.integers(1, 50))
        D = 8
        x = rng.standard_normal(n) * 3
        v = rng.standard_normal((n, D))
        P = int(rng.integers(1, 8))
        cuts = np.sort(rng.integers(0, n + 1, size=P - 1))
        bounds = np.concatenate([[0], cuts, [n]])
        pm = np.full((1, 1, 1, P), -np.inf); pl = np.zeros((1, 1, 1, P))
        po = np.zeros((1, 1, 1, P, D))
        for c in range(P):
            a, b = bounds[c], bounds[c + 1]
            if b > a:
                m = x[a:b].max()
                e = np.exp(x[a:b] - m)
                pm[0, 0, 0, c], pl[0, 0, 0, c] = m, e.sum()
                po[0, 0, 0, c] = e @ v[a:b]
        out = orc.merge(pm, pl, po)
        assert np.allclose(out[0, 0, 0], softmax(x) @ v, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------- golden ---

def _golden_inputs(g):
    f16 = lambda a: np.array(a, dtype=np.float64).astype(np.float16)
    T, N, Hq, Hkv, D = g["T"], g["N"], g["Hq"], g["Hkv"], g["D"]
    inp = dict(q_idx=f16(g["q_idx"]).reshape(1, T, -1),
               K_idx=f16(g["K_idx"]).reshape(1, N, -1),
               q=np.array(g["q"], dtype=np.float32).reshape(1, T, Hq, D),
               Kq=np.array(g["Kq"], dtype=np.int8).reshape(1, N, Hkv, D),
               Ksc=f16(g["Ksc"]).reshape(1, N, Hkv, D // 32),
               Vq=np.array(g["Vq"], dtype=np.int8).reshape(1, N, Hkv, D),
               Vsc=f16(g["Vsc"]).reshape(1, N, Hkv, D // 32),
               k=g["k"], pos0=g["pos0"], dense_max=g["dense_max"], cap=g["cap"])
    return inp


def _expand(spec, shape):
    """Golden files list only the nonzero entries: {"flat index": value}."""
    a = np.zeros(int(np.prod(shape)))
    for key, val in spec.items():
        a[int(key)] = val
    return a.reshape(shape)


def load_golden():
    cases = []
    for path in sorted(glob.glob(os.path.join(HERE, "golden", "*.json"))):
        with open(path) as f:
            g = json.load(f)
        T, N, Hq, Hkv, D, di = g["T"], g["N"], g["Hq"], g["Hkv"], g["D"], g["di"]
        for name, shape in (("q_idx", (T, di)), ("K_idx", (N, di)), ("q", (T, Hq, D)),
                            ("Kq", (N, Hkv, D)), ("Ksc", (N, Hkv, D // 32)),
                            ("Vq", (N, Hkv, D)), ("Vsc", (N, Hkv, D // 32))):
            if isinstance(g[name], dict):
                g[name] = _expand(g[name], shape).tolist()
        g["_path"] = path
        cases.append(g)
    return cases


def pin_golden(orc):
    cases = load_golden()
    assert cases, "no golden cases found"
    for g in cases:
        inp = _golden_inputs(g)
        res = orc.run(inp, P=g["P"], scale=g["scale"])
        exp = g["expect"]
        n = exp["n_sel"]
        assert list(res["n_sel"][0]) == n, g["_path"]
        for t in range(g["T"]):
            assert list(res["ids"][0, t, : n[t]]) == exp["ids"][t], g["_path"]
            assert (res["ids"][0, t, n[t]:] == -1).all()
        out = np.array(exp["out"], dtype=np.float64).reshape(res["out"].shape)
        assert np.allclose(res["out"], out, rtol=0, atol=float(exp["atol"])), g["_path"]
        if "m" in exp:
            assert np.allclose(res["pm"].ravel(), np.array(exp["m"], float),
                               rtol=0, atol=1e-15)
            assert np.allclose(res["pl"].ravel(), np.array(exp["l"], float),
                               rtol=0, atol=1e-15)


# -------------------------------------------------------- KV quantiser ---

_F16_TABLE = None


def _f16_table():
    """All finite non-negative binary16 values (ascending) as Fractions, with
    their bit patterns (numpy's binary16 decoding)."""
    global _F16_TABLE
    if _F16_TABLE is None:
        bits = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16)
        vals = bits.view(np.float16).astype(np.float64)
        _F16_TABLE = ([Fraction(float(v)) for v in vals], bits)
    return _F16_TABLE


def _exact_scale_bits(a: Fraction) -> int:
    """Bit pattern of the binary16 value nearest to a / 127, ties to even."""
    vals, bits = _f16_table()
    t = a / 127
    i = bisect.bisect_left(vals, t)
    cands = [j for j in (i - 1, i, i + 1) if 0 <= j < len(vals)]
    best = min(cands, key=lambda j: (abs(vals[j] - t), int(bits[j]) & 1))
    return int(bits[best])


def _exact_quant(x: np.ndarray):
    """Reference quantisation of one float32 row: per 32-block absmax scale
    fp16(a / 127) and codes round(x / s) (ties to even) clamped to +-127."""
    codes = np.zeros(x.size, dtype=np.int8)
    scales = np.zeros(x.size // 32, dtype=np.uint16)
    vals, _ = _f16_table()
    for blk in range(x.size // 32):
        xb = [Fraction(float(v)) for v in x[32 * blk: 32 * blk + 32]]
        a = max(abs(v) for v in xb)
        hb = _exact_scale_bits(a)
        scales[blk] = hb
        sv = vals[hb]
        for e, v in enumerate(xb):
            c = round(v / sv) if sv != 0 else 0       # Fraction rounds half to even
            codes[32 * blk + e] = max(-127, min(127, c))
    return codes, scales


def pin_quantiser_exact(orc):
    """Codes and scales of random rows at magnitudes from fp16-subnormal
    scales (where the +-127 clamp engages) to large ones equal the exact
    rational reference."""
    rng = np.random.default_rng(71)
    for mag in (3e-9, 2e-7, 1e-4, 1.0, 37.0, 3e5):
        for _ in range(3):
            x = (rng.normal(size=64) * mag).astype(np.float32)
            x[rng.integers(0, 64, 3)] = 0.0
            got_c, got_s = orc.quant_row(x)
            ref_c, ref_s = _exact_quant(x)
            assert np.array_equal(got_s, ref_s), (mag, got_s, ref_s)
            assert np.array_equal(got_c, ref_c), mag
    # an all-zero block: scale 0, codes 0
    c, s_ = orc.quant_row(np.zeros(32, dtype=np.float32))
    assert not c.any() and not s_.any()


def pin_quantiser_ties(orc):
    """Exact ties x / s = n + 1/2 go to the even code, for both signs; the
    block maximum 127 * s gives code +-127 and scale s exactly."""
    for s in (0.5, 2.0 ** -10, 3.0, 0.0625 * 3):
        x = np.zeros(32, dtype=np.float32)
        x[0] = 127 * s
        halves = [0.5, 1.5, 2.5, 3.5, 10.5, 125.5]
        for i, hv in enumerate(halves):
            x[1 + i] = hv * s
            x[1 + len(halves) + i] = -hv * s
        c, sc = orc.quant_row(x)
        assert float(np.array([sc[0]], np.uint16).view(np.float16)[0]) == s
        assert c[0] == 127
        for i, hv in enumerate(halves):
            lo = int(math.floor(hv))
            even = lo if lo % 2 == 0 else lo + 1
            assert c[1 + i] == even, (s, hv, c[1 + i])
            assert c[1 + len(halves) + i] == -even, (s, -hv)


def pin_append_placement(orc):
    """kv_append writes exactly cells pos0 .. pos0+T-1: K and V rows are the
    per-row quantisation of the new rows, index keys are numpy's binary16
    rounding, every other cell is untouched."""
    rng = np.random.default_rng(73)
    B, N, T, Hkv, D, di, pos0 = 2, 12, 3, 2, 64, 16, 5
    Kq = rng.integers(-127, 128, size=(B, N, Hkv, D)).astype(np.int8)
    Vq = rng.integers(-127, 128, size=(B, N, Hkv, D)).astype(np.int8)
    Ksc = rng.integers(0, 0x7000, size=(B, N, Hkv, D // 32)).astype(np.uint16)
    Vsc = rng.integers(0, 0x7000, size=(B, N, Hkv, D // 32)).astype(np.uint16)
    Kix = rng.integers(0, 0x7000, size=(B, N, di)).astype(np.uint16)
    k_new = rng.normal(size=(B, T, Hkv, D)).astype(np.float32)
    v_new = (rng.normal(size=(B, T, Hkv, D)) * 5).astype(np.float32)
    i_new = rng.normal(size=(B, T, di)).astype(np.float32)
    oK, oKs, oV, oVs, oI = orc.kv_append(k_new, v_new, i_new, Kq, Ksc, Vq, Vsc, Kix,
                                         pos0=pos0)
    keep = np.ones(N, bool)
    keep[pos0:pos0 + T] = False
    for a, o in ((Kq, oK), (Ksc, oKs), (Vq, oV), (Vsc, oVs), (Kix, oI)):
        assert np.array_equal(np.asarray(a)[:, keep], np.asarray(o)[:, keep])
    for b in range(B):
        for t in range(T):
            assert np.array_equal(oI[b, pos0 + t], i_new[b, t].astype(np.float16).view(np.uint16))
            for g in range(Hkv):
                for new, codes, scales in ((k_new, oK, oKs), (v_new, oV, oVs)):
                    rc, rs = _exact_quant(new[b, t, g])
                    assert np.array_equal(codes[b, pos0 + t, g], rc)
                    assert np.array_equal(scales[b, pos0 + t, g], rs)


def pin_gate(orc):
    """The gated merge is the plain merge times scipy's logistic sigmoid of
    the gate, elementwise; gate 0 halves the output exactly, large gates
    pass it through or shut it."""
    from scipy.special import expit
    rng = np.random.default_rng(83)
    B, T, Hq, P, D = 2, 3, 4, 5, 32
    pm = rng.normal(size=(B, T, Hq, P)) * 3
    pm[0, 1, 2, :2] = -np.inf                                   # empty chunks
    pl = rng.uniform(0.5, 4, size=(B, T, Hq, P))
    pl[np.isneginf(pm)] = 0
    po = rng.normal(size=(B, T, Hq, P, D))
    po[np.isneginf(pm)] = 0
    gate = rng.normal(size=(B, T, Hq, D)) * 4
    gate[0, 0, 0, :3] = (0.0, 60.0, -60.0)
    plain = orc.merge(pm, pl, po)
    got = orc.merge_gated(pm, pl, po, gate)
    assert np.allclose(got, plain * expit(gate), rtol=1e-13, atol=0)
    assert got[0, 0, 0, 0] == plain[0, 0, 0, 0] * 0.5
    assert abs(got[0, 0, 0, 1] - plain[0, 0, 0, 1]) <= 1e-25 * abs(plain[0, 0, 0, 1]) + 1e-300
    assert abs(got[0, 0, 0, 2]) <= 1e-25 * abs(plain[0, 0, 0, 2])
    g16 = gate.astype(np.float16)
    assert np.allclose(orc.merge_gated(pm, pl, po, g16),
                       plain * expit(g16.astype(np.float64)), rtol=1e-13, atol=0)


ALL_PINS = [
    pin_half_decode_exhaustive,
    pin_half_encode,
    pin_scores_matmul,
    pin_topk_bruteforce,
    pin_dense_boundary,
    pin_topk_invariants,
    pin_attention_bruteforce,
    pin_closed_forms,
    pin_k_covers_all,
    pin_split_invariance,
    pin_merge_textbook,
    pin_golden,
    pin_quantiser_exact,
    pin_quantiser_ties,
    pin_append_placement,
    pin_gate,
]
