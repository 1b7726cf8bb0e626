"""ctypes front end of the double-precision CPU oracle in ``qsa_oracle.c``.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it, and it imports nothing from the HIP package: inputs arrive as plain
numpy arrays (the same seeded arrays the GPU side receives) and every result
is computed by the C code next to this file.

All arrays carry a leading batch dimension B of independent problems; the C
oracle handles one problem at a time and this wrapper loops over B.

Layouts (row-major):
  q_idx [B][T][di] fp16        K_idx [B][N][di] fp16
  q     [B][T][Hq][D] f32|f16  Kq, Vq [B][N][Hkv][D] int8
  Ksc, Vsc [B][N][Hkv][D/32] fp16
  ids   [B][T][cap] int32      n_sel [B][T] int32
  pm, pl [B][T][Hq][P] f64     po [B][T][Hq][P][D] f64     out [B][T][Hq][D] f64
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qsa_oracle.c")
LIB = os.path.join(HERE, "libqsa_oracle.so")

CFLAGS = ("-O2", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11")


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (no FMA contraction, as a plain reference)."""
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _needs_build(src: str, lib: str) -> bool:
    return (not os.path.exists(lib)) or os.path.getmtime(lib) < os.path.getmtime(src)


_P = ctypes.c_void_p
_I = ctypes.c_int


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _bits16(a: np.ndarray) -> np.ndarray:
    """fp16 array (or its uint16 bit pattern) -> contiguous uint16 bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


class Oracle:
    """One loaded build of the oracle library (the default, or a test mutant)."""

    def __init__(self, libpath: str = LIB, src: str = SRC):
        if libpath == LIB and _needs_build(src, libpath):
            build(src, libpath)
        self.path = libpath
        lib = ctypes.CDLL(libpath)
        lib.qo_half_to_double.argtypes = [ctypes.c_uint16]
        lib.qo_half_to_double.restype = ctypes.c_double
        lib.qo_double_to_half.argtypes = [ctypes.c_double]
        lib.qo_double_to_half.restype = ctypes.c_uint16
        lib.qo_index_topk.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]
        lib.qo_index_topk.restype = _I
        lib.qo_attend.argtypes = [_I, _I, _I, _I, _I, _I, ctypes.c_double, _I, _P,
                                  _P, _P, _P, _P, _P, _P, _P, _P, _P]
        lib.qo_attend.restype = _I
        lib.qo_merge.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P]
        lib.qo_merge.restype = _I
        lib.qo_merge_gated.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P]
        lib.qo_merge_gated.restype = _I
        lib.qo_quant_row.argtypes = [_I, _P, _P, _P]
        lib.qo_quant_row.restype = _I
        lib.qo_kv_append.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]
        lib.qo_kv_append.restype = _I
        self.lib = lib

    # ------------------------------------------------------------- fp16 ---
    def half_to_double(self, bits) -> np.ndarray:
        bits = np.asarray(bits, dtype=np.uint16).ravel()
        f = self.lib.qo_half_to_double
        return np.array([f(int(b)) for b in bits], dtype=np.float64)

    def double_to_half(self, x) -> np.ndarray:
        x = np.asarray(x, dtype=np.float64)
        f = self.lib.qo_double_to_half
        flat = np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16)
        return flat.reshape(x.shape)

    # ---------------------------------------------------- index + top-k ---
    def index_topk(self, q_idx, K_idx, *, k: int, pos0: int, dense_max: int,
                   cap: int, want_scores: bool = False):
        q_idx = _bits16(q_idx)
        K_idx = _bits16(K_idx)
        B, T, di = q_idx.shape
        B2, N, di2 = K_idx.shape
        assert B == B2 and di == di2
        ids = np.empty((B, T, cap), dtype=np.int32)
        n_sel = np.empty((B, T), dtype=np.int32)
        scores = np.empty((B, T, N), dtype=np.float64) if want_scores else None
        for b in range(B):
            qb = np.ascontiguousarray(q_idx[b])
            kb = np.ascontiguousarray(K_idx[b])
            ib = np.empty((T, cap), dtype=np.int32)
            nb = np.empty((T,), dtype=np.int32)
            sb = np.empty((T, N), dtype=np.float64) if want_scores else None
            rc = self.lib.qo_index_topk(T, N, di, k, pos0, dense_max, cap,
                                        _ptr(qb), _ptr(kb), _ptr(ib), _ptr(nb),
                                        _ptr(sb) if want_scores else None)
            if rc != 0:
                raise ValueError("oracle qo_index_topk rejected its arguments")
            ids[b], n_sel[b] = ib, nb
            if want_scores:
                scores[b] = sb
        return (ids, n_sel, scores) if want_scores else (ids, n_sel)

    # ----------------------------------------------------------- attend ---
    def attend(self, q, Kq, Ksc, Vq, Vsc, ids, n_sel, *, P: int, scale: float):
        q = np.ascontiguousarray(q)
        if q.dtype == np.float16:
            q_is_f16 = 1
        else:
            assert q.dtype == np.float32, q.dtype
            q_is_f16 = 0
        B, T, Hq, D = q.shape
        _, N, Hkv, D2 = Kq.shape
        assert D == D2 and Kq.dtype == np.int8 and Vq.dtype == np.int8
        Ksc, Vsc = _bits16(Ksc), _bits16(Vsc)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        n_sel = np.ascontiguousarray(n_sel, dtype=np.int32)
        cap = ids.shape[-1]
        pm = np.empty((B, T, Hq, P), dtype=np.float64)
        pl = np.empty((B, T, Hq, P), dtype=np.float64)
        po = np.empty((B, T, Hq, P, D), dtype=np.float64)
        for b in range(B):
            qb = np.ascontiguousarray(q[b])
            kq, ks = np.ascontiguousarray(Kq[b]), np.ascontiguousarray(Ksc[b])
            vq, vs = np.ascontiguousarray(Vq[b]), np.ascontiguousarray(Vsc[b])
            ib, nb = np.ascontiguousarray(ids[b]), np.ascontiguousarray(n_sel[b])
            mb = np.empty((T, Hq, P)); lb = np.empty((T, Hq, P))
            ob = np.empty((T, Hq, P, D))
            rc = self.lib.qo_attend(T, Hq, Hkv, D, P, cap, float(scale), q_is_f16,
                                    _ptr(qb), _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs),
                                    _ptr(ib), _ptr(nb), _ptr(mb), _ptr(lb), _ptr(ob))
            if rc != 0:
                raise ValueError("oracle qo_attend rejected its arguments")
            pm[b], pl[b], po[b] = mb, lb, ob
        return pm, pl, po

    # ------------------------------------------------------------ merge ---
    def merge(self, pm, pl, po) -> np.ndarray:
        pm = np.ascontiguousarray(pm, dtype=np.float64)
        pl = np.ascontiguousarray(pl, dtype=np.float64)
        po = np.ascontiguousarray(po, dtype=np.float64)
        B, T, Hq, P, D = po.shape
        out = np.empty((B, T, Hq, D), dtype=np.float64)
        for b in range(B):
            ob = np.empty((T, Hq, D))
            rc = self.lib.qo_merge(T, Hq, P, D, _ptr(np.ascontiguousarray(pm[b])),
                                   _ptr(np.ascontiguousarray(pl[b])),
                                   _ptr(np.ascontiguousarray(po[b])), _ptr(ob))
            if rc != 0:
                raise ValueError("oracle qo_merge rejected its arguments")
            out[b] = ob
        return out

    def merge_gated(self, pm, pl, po, gate) -> np.ndarray:
        """Merge, then the elementwise sigmoid output gate (gate [B][T][Hq][D],
        fp32 or fp16)."""
        pm = np.ascontiguousarray(pm, dtype=np.float64)
        pl = np.ascontiguousarray(pl, dtype=np.float64)
        po = np.ascontiguousarray(po, dtype=np.float64)
        gate = np.ascontiguousarray(np.asarray(gate).astype(np.float64))
        B, T, Hq, P, D = po.shape
        out = np.empty((B, T, Hq, D), dtype=np.float64)
        for b in range(B):
            ob = np.empty((T, Hq, D))
            rc = self.lib.qo_merge_gated(T, Hq, P, D, _ptr(np.ascontiguousarray(pm[b])),
                                         _ptr(np.ascontiguousarray(pl[b])),
                                         _ptr(np.ascontiguousarray(po[b])),
                                         _ptr(np.ascontiguousarray(gate[b])), _ptr(ob))
            if rc != 0:
                raise ValueError("oracle qo_merge_gated rejected its arguments")
            out[b] = ob
        return out

    # -------------------------------------------------------- KV append ---
    def quant_row(self, x):
        """One float32 row (length a multiple of 32) -> (int8 codes, fp16
        scale bits)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        codes = np.empty(x.shape, dtype=np.int8)
        scales = np.empty((x.size // 32,), dtype=np.uint16)
        if self.lib.qo_quant_row(x.size, _ptr(x), _ptr(codes), _ptr(scales)) != 0:
            raise ValueError("oracle qo_quant_row rejected its arguments")
        return codes, scales

    def kv_append(self, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx, *, pos0: int):
        """Returns copies of the dense caches (Kq, Ksc, Vq, Vsc as int8 / fp16
        bits, K_idx as fp16 bits) with the T new tokens of every problem
        quantised in at positions pos0 .. pos0+T-1."""
        k_new = np.ascontiguousarray(k_new, dtype=np.float32)
        v_new = np.ascontiguousarray(v_new, dtype=np.float32)
        kidx_new = np.ascontiguousarray(kidx_new, dtype=np.float32)
        B, T, Hkv, D = k_new.shape
        di = kidx_new.shape[-1]
        Kq, Vq = np.array(Kq, dtype=np.int8), np.array(Vq, dtype=np.int8)
        Ksc, Vsc, K_idx = (np.array(_bits16(a)) for a in (Ksc, Vsc, K_idx))
        N = Kq.shape[1]
        for b in range(B):
            kq, ks = np.ascontiguousarray(Kq[b]), np.ascontiguousarray(Ksc[b])
            vq, vs = np.ascontiguousarray(Vq[b]), np.ascontiguousarray(Vsc[b])
            ki = np.ascontiguousarray(K_idx[b])
            rc = self.lib.qo_kv_append(T, N, Hkv, D, di, pos0,
                                       _ptr(np.ascontiguousarray(k_new[b])),
                                       _ptr(np.ascontiguousarray(v_new[b])),
                                       _ptr(np.ascontiguousarray(kidx_new[b])),
                                       _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs), _ptr(ki))
            if rc != 0:
                raise ValueError("oracle qo_kv_append rejected its arguments")
            Kq[b], Ksc[b], Vq[b], Vsc[b], K_idx[b] = kq, ks, vq, vs, ki
        return Kq, Ksc, Vq, Vsc, K_idx

    # ------------------------------------------------------- whole path ---
    def run(self, inp: dict, *, P: int, scale: float | None = None):
        """index_topk -> attend -> merge on one input dict (see datagen)."""
        ids, n_sel = self.index_topk(inp["q_idx"], inp["K_idx"], k=inp["k"],
                                     pos0=inp["pos0"], dense_max=inp["dense_max"],
                                     cap=inp["cap"])
        D = inp["q"].shape[-1]
        sc = (1.0 / np.sqrt(D)) if scale is None else scale
        pm, pl, po = self.attend(inp["q"], inp["Kq"], inp["Ksc"], inp["Vq"],
                                 inp["Vsc"], ids, n_sel, P=P, scale=sc)
        out = self.merge(pm, pl, po)
        return dict(ids=ids, n_sel=n_sel, pm=pm, pl=pl, po=po, out=out)


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
