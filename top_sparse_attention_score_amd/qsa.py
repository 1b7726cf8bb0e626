"""Thin ctypes binding of libqsa.so (the C ABI in include/qsa.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, builds the C descriptor, and passes raw device pointers and
torch's current HIP stream to the library.  All computation happens in the
library's HIP kernels.  There is no fallback: if libqsa.so is missing or a
call is rejected, a QsaError is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_F32 = 0
QSA_F16 = 1
# qsa_attend kernel families (qsa_attend_algo)
QSA_ATTEND_AUTO = 0
QSA_ATTEND_MATRIX = 1
QSA_ATTEND_VECTOR = 2
# bytes of the fixed workspace of qsa_index_topk_noalloc (include/qsa.h)
QSA_NOALLOC_WORKSPACE_BYTES = 64 << 20

_c_int, _c_ll, _c_float, _vp = ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_void_p


class QsaError(RuntimeError):
    pass


class IndexDesc(ctypes.Structure):
    _fields_ = [("batch", _c_int), ("T", _c_int), ("n_cells", _c_int), ("d_idx", _c_int),
                ("k", _c_int), ("pos0", _c_int), ("dense_max", _c_int), ("ids_cap", _c_int)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", _c_int), ("T", _c_int), ("Hq", _c_int), ("Hkv", _c_int),
                ("D", _c_int), ("P", _c_int), ("ids_cap", _c_int), ("n_cells", _c_int),
                ("scale", _c_float), ("q_dtype", _c_int), ("out_dtype", _c_int),
                ("algo", _c_int), ("kq_cell_stride", _c_ll), ("ksc_cell_stride", _c_ll),
                ("vq_cell_stride", _c_ll), ("vsc_cell_stride", _c_ll),
                ("kq_batch_stride", _c_ll), ("ksc_batch_stride", _c_ll),
                ("vq_batch_stride", _c_ll), ("vsc_batch_stride", _c_ll)]


class AppendDesc(ctypes.Structure):
    _fields_ = [("batch", _c_int), ("T", _c_int), ("n_cells", _c_int), ("pos0", _c_int),
                ("Hkv", _c_int), ("D", _c_int), ("d_idx", _c_int), ("reserved", _c_int),
                ("kq_cell_stride", _c_ll), ("ksc_cell_stride", _c_ll),
                ("vq_cell_stride", _c_ll), ("vsc_cell_stride", _c_ll),
                ("kq_batch_stride", _c_ll), ("ksc_batch_stride", _c_ll),
                ("vq_batch_stride", _c_ll), ("vsc_batch_stride", _c_ll)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqsa.so once (raises QsaError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QsaError(f"{LIB_PATH} is missing: build it with "
                           "top_sparse_attention_score_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.qsa_status_string.argtypes = [_c_int]
        L.qsa_status_string.restype = ctypes.c_char_p
        L.qsa_version.restype = _c_int
        L.qsa_index_topk_workspace.argtypes = [ctypes.POINTER(IndexDesc)]
        L.qsa_index_topk_workspace.restype = ctypes.c_size_t
        L.qsa_index_topk.argtypes = [ctypes.POINTER(IndexDesc), _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]
        L.qsa_index_topk.restype = _c_int
        L.qsa_index_topk_noalloc.argtypes = [ctypes.POINTER(IndexDesc), _vp, _vp, _vp, _vp,
                                             _vp]
        L.qsa_index_topk_noalloc.restype = _c_int
        L.qsa_partials_floats.argtypes = [ctypes.POINTER(AttnDesc)]
        L.qsa_partials_floats.restype = ctypes.c_size_t
        L.qsa_attend.argtypes = [ctypes.POINTER(AttnDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp]
        L.qsa_attend.restype = _c_int
        L.qsa_merge.argtypes = [ctypes.POINTER(AttnDesc), _vp, _vp, _vp]
        L.qsa_merge.restype = _c_int
        L.qsa_merge_gated.argtypes = [ctypes.POINTER(AttnDesc), _vp, _vp, _vp, _vp]
        L.qsa_merge_gated.restype = _c_int
        L.qsa_attend_merge.argtypes = [ctypes.POINTER(AttnDesc)] + [_vp] * 10
        L.qsa_attend_merge.restype = _c_int
        L.qsa_kv_append.argtypes = [ctypes.POINTER(AppendDesc), _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp]
        L.qsa_kv_append.restype = _c_int
        L.qsa_decode_window_workspace.argtypes = [ctypes.POINTER(IndexDesc),
                                                  ctypes.POINTER(AttnDesc)]
        L.qsa_decode_window_workspace.restype = ctypes.c_size_t
        L.qsa_decode_window.argtypes = [ctypes.POINTER(AppendDesc), ctypes.POINTER(IndexDesc),
                                        ctypes.POINTER(AttnDesc)] + [_vp] * 15 + \
                                       [ctypes.c_size_t, _vp]
        L.qsa_decode_window.restype = _c_int
        L.qsa_step_workspace.argtypes = [ctypes.POINTER(IndexDesc), ctypes.POINTER(AttnDesc)]
        L.qsa_step_workspace.restype = ctypes.c_size_t
        L.qsa_step.argtypes = [ctypes.POINTER(AppendDesc), ctypes.POINTER(IndexDesc),
                               ctypes.POINTER(AttnDesc)] + [_vp] * 15 + [ctypes.c_size_t, _vp]
        L.qsa_step.restype = _c_int
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().qsa_status_string(code).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise QsaError(f"{what}: {status_string(code)} ({code})")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


# ------------------------------------------------------ size validation ---
#
# The library receives raw pointers and cannot see how large a buffer is; a
# tensor shorter than the descriptor says would be read or written past its
# end on the GPU.  Every call therefore checks, before anything is enqueued,
# that each tensor's storage holds at least the bytes the descriptor
# addresses from its data pointer on, and then that every tensor is on the
# GPU.

def _avail(t) -> int:
    st = t.untyped_storage()
    return st.nbytes() - (t.data_ptr() - st.data_ptr())


def _need(t, nbytes: int, what: str, optional: bool = False) -> None:
    if t is None:
        if optional:
            return
        raise QsaError(f"{what}: missing tensor")
    if _avail(t) < nbytes:
        raise QsaError(f"{what}: tensor holds {_avail(t)} bytes from its start, "
                       f"the call addresses {nbytes}")


def _on_gpu(what: str, *tensors) -> None:
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise QsaError(f"{what}: not a GPU tensor")


def _esize(dtype_code: int) -> int:
    return 2 if dtype_code == QSA_F16 else 4


def _cache_bytes(d, name: str, per_cell: int, cell_dense: int) -> int:
    cs = getattr(d, f"{name}_cell_stride") or cell_dense
    bs = getattr(d, f"{name}_batch_stride") or d.n_cells * cs
    return (d.batch - 1) * bs + (d.n_cells - 1) * cs + per_cell


def _check_cache(d, Kq, Ksc, Vq, Vsc) -> None:
    codes, scales = d.Hkv * d.D, d.Hkv * (d.D // 32) * 2
    _need(Kq, _cache_bytes(d, "kq", codes, codes), "Kq")
    _need(Ksc, _cache_bytes(d, "ksc", scales, scales), "Ksc")
    _need(Vq, _cache_bytes(d, "vq", codes, codes), "Vq")
    _need(Vsc, _cache_bytes(d, "vsc", scales, scales), "Vsc")


def _check_index(d, q_idx, K_idx, ids, n_sel) -> None:
    _need(q_idx, d.batch * d.T * d.d_idx * 2, "q_idx")
    _need(K_idx, d.batch * d.n_cells * d.d_idx * 2, "K_idx")
    _need(ids, d.batch * d.T * d.ids_cap * 4, "ids")
    _need(n_sel, d.batch * d.T * 4, "n_sel")


def _check_attn(d, q, ids, n_sel, gate=None, out=None, gate_optional=True) -> None:
    rows = d.batch * d.T * d.Hq * d.D
    _need(q, rows * _esize(d.q_dtype), "q")
    _need(ids, d.batch * d.T * d.ids_cap * 4, "ids")
    _need(n_sel, d.batch * d.T * 4, "n_sel")
    _need(gate, rows * _esize(d.q_dtype), "gate", optional=gate_optional)
    if out is not None:
        _need(out, rows * _esize(d.out_dtype), "out")


def _check_append(d, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx) -> None:
    rows = d.batch * d.T * d.Hkv * d.D * 4
    _need(k_new, rows, "k_new")
    _need(v_new, rows, "v_new")
    _need(kidx_new, d.batch * d.T * d.d_idx * 4, "kidx_new", optional=True)
    _check_cache(d, Kq, Ksc, Vq, Vsc)
    if kidx_new is not None:
        _need(K_idx, d.batch * d.n_cells * d.d_idx * 2, "K_idx")


# ----------------------------------------------------------- descriptors ---

def index_desc(*, batch: int, T: int, n_cells: int, d_idx: int, k: int, pos0: int,
               dense_max: int, ids_cap: int) -> IndexDesc:
    return IndexDesc(batch, T, n_cells, d_idx, k, pos0, dense_max, ids_cap)


def attn_desc(*, batch: int, T: int, Hq: int, Hkv: int, D: int, P: int, ids_cap: int,
              n_cells: int, scale: float | None = None, q_dtype: int = QSA_F32,
              out_dtype: int = QSA_F32, strides: dict | None = None,
              algo: int = 0) -> AttnDesc:
    """Attention descriptor; `strides` may set any of the *_cell_stride /
    *_batch_stride fields (bytes); unset ones keep the dense default.
    scale None passes 0, for which the library uses its default."""
    sc = 0.0 if scale is None else float(scale)
    d = AttnDesc(batch, T, Hq, Hkv, D, P, ids_cap, n_cells, sc, q_dtype, out_dtype, algo)
    for key, val in (strides or {}).items():
        setattr(d, key, int(val))
    return d


def append_desc(*, batch: int, T: int, n_cells: int, pos0: int, Hkv: int, D: int, d_idx: int,
                strides: dict | None = None) -> AppendDesc:
    """KV-append descriptor; `strides` as for attn_desc."""
    d = AppendDesc(batch, T, n_cells, pos0, Hkv, D, d_idx, 0)
    for key, val in (strides or {}).items():
        setattr(d, key, int(val))
    return d


def qsa_index_topk_workspace(desc: IndexDesc) -> int:
    return int(lib().qsa_index_topk_workspace(ctypes.byref(desc)))


def qsa_partials_floats(desc: AttnDesc) -> int:
    return int(lib().qsa_partials_floats(ctypes.byref(desc)))


# ----------------------------------------------------------------- calls ---

def qsa_index_topk(desc: IndexDesc, q_idx, K_idx, ids, n_sel, ws, stream=None) -> None:
    _check_index(desc, q_idx, K_idx, ids, n_sel)
    _on_gpu("qsa_index_topk", q_idx, K_idx, ids, n_sel, ws)
    _check(lib().qsa_index_topk(ctypes.byref(desc), _ptr(q_idx), _ptr(K_idx), _ptr(ids),
                                _ptr(n_sel), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "qsa_index_topk")


def qsa_index_topk_noalloc(desc: IndexDesc, q_idx, K_idx, ids, n_sel, stream=None) -> None:
    _check_index(desc, q_idx, K_idx, ids, n_sel)
    _on_gpu("qsa_index_topk_noalloc", q_idx, K_idx, ids, n_sel)
    _check(lib().qsa_index_topk_noalloc(ctypes.byref(desc), _ptr(q_idx), _ptr(K_idx), _ptr(ids),
                                        _ptr(n_sel), _stream(stream)), "qsa_index_topk_noalloc")


def qsa_attend(desc: AttnDesc, q, Kq, Ksc, Vq, Vsc, ids, n_sel, partials,
               stream=None) -> None:
    _check_attn(desc, q, ids, n_sel)
    _check_cache(desc, Kq, Ksc, Vq, Vsc)
    _need(partials, qsa_partials_floats(desc) * 4, "partials")
    _on_gpu("qsa_attend", q, Kq, Ksc, Vq, Vsc, ids, n_sel, partials)
    _check(lib().qsa_attend(ctypes.byref(desc), _ptr(q), _ptr(Kq), _ptr(Ksc), _ptr(Vq),
                            _ptr(Vsc), _ptr(ids), _ptr(n_sel), _ptr(partials),
                            _stream(stream)), "qsa_attend")


def qsa_merge(desc: AttnDesc, partials, out, stream=None) -> None:
    _need(partials, qsa_partials_floats(desc) * 4, "partials")
    _need(out, desc.batch * desc.T * desc.Hq * desc.D * _esize(desc.out_dtype), "out")
    _on_gpu("qsa_merge", partials, out)
    _check(lib().qsa_merge(ctypes.byref(desc), _ptr(partials), _ptr(out), _stream(stream)),
           "qsa_merge")


def qsa_merge_gated(desc: AttnDesc, partials, gate, out, stream=None) -> None:
    _need(partials, qsa_partials_floats(desc) * 4, "partials")
    rows = desc.batch * desc.T * desc.Hq * desc.D
    _need(gate, rows * _esize(desc.q_dtype), "gate", optional=True)
    _need(out, rows * _esize(desc.out_dtype), "out")
    _on_gpu("qsa_merge_gated", partials, gate, out)
    _check(lib().qsa_merge_gated(ctypes.byref(desc), _ptr(partials), _ptr(gate), _ptr(out),
                                 _stream(stream)), "qsa_merge_gated")


def qsa_attend_merge(desc: AttnDesc, q, Kq, Ksc, Vq, Vsc, ids, n_sel, gate, out,
                     stream=None) -> None:
    _check_attn(desc, q, ids, n_sel, gate, out)
    _check_cache(desc, Kq, Ksc, Vq, Vsc)
    _on_gpu("qsa_attend_merge", q, Kq, Ksc, Vq, Vsc, ids, n_sel, gate, out)
    _check(lib().qsa_attend_merge(ctypes.byref(desc), _ptr(q), _ptr(Kq), _ptr(Ksc), _ptr(Vq),
                                  _ptr(Vsc), _ptr(ids), _ptr(n_sel), _ptr(gate), _ptr(out),
                                  _stream(stream)), "qsa_attend_merge")


def qsa_kv_append(desc: AppendDesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx,
                  stream=None) -> None:
    _check_append(desc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx)
    _on_gpu("qsa_kv_append", k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx)
    _check(lib().qsa_kv_append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(kidx_new),
                               _ptr(Kq), _ptr(Ksc), _ptr(Vq), _ptr(Vsc), _ptr(K_idx),
                               _stream(stream)), "qsa_kv_append")


def _check_step(pdesc, idesc, adesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx, q_idx,
                q, gate, ids, n_sel, out, ws, ws_need) -> None:
    _check_append(pdesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx)
    _check_index(idesc, q_idx, K_idx, ids, n_sel)
    _check_attn(adesc, q, ids, n_sel, gate, out)
    _check_cache(adesc, Kq, Ksc, Vq, Vsc)
    if ws_need:
        _need(ws, ws_need, "workspace")
    _on_gpu("the step", k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx, q_idx, q, gate, ids,
            n_sel, out, ws)


def qsa_decode_window_workspace(idesc: IndexDesc, adesc: AttnDesc) -> int:
    return int(lib().qsa_decode_window_workspace(ctypes.byref(idesc), ctypes.byref(adesc)))


def qsa_decode_window(pdesc: AppendDesc, idesc: IndexDesc, adesc: AttnDesc, k_new, v_new,
                      kidx_new, Kq, Ksc, Vq, Vsc, K_idx, q_idx, q, gate, ids, n_sel, out, ws,
                      stream=None) -> None:
    _check_step(pdesc, idesc, adesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx, q_idx, q,
                gate, ids, n_sel, out, ws, qsa_decode_window_workspace(idesc, adesc))
    _check(lib().qsa_decode_window(
        ctypes.byref(pdesc), ctypes.byref(idesc), ctypes.byref(adesc), _ptr(k_new), _ptr(v_new),
        _ptr(kidx_new), _ptr(Kq), _ptr(Ksc), _ptr(Vq), _ptr(Vsc), _ptr(K_idx), _ptr(q_idx),
        _ptr(q), _ptr(gate), _ptr(ids), _ptr(n_sel), _ptr(out), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
        "qsa_decode_window")


def qsa_step_workspace(idesc: IndexDesc, adesc: AttnDesc) -> int:
    return int(lib().qsa_step_workspace(ctypes.byref(idesc), ctypes.byref(adesc)))


def qsa_step(pdesc: AppendDesc, idesc: IndexDesc, adesc: AttnDesc, k_new, v_new, kidx_new, Kq,
             Ksc, Vq, Vsc, K_idx, q_idx, q, gate, ids, n_sel, out, ws, stream=None) -> None:
    _check_step(pdesc, idesc, adesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx, q_idx, q,
                gate, ids, n_sel, out, ws, qsa_step_workspace(idesc, adesc))
    _check(lib().qsa_step(
        ctypes.byref(pdesc), ctypes.byref(idesc), ctypes.byref(adesc), _ptr(k_new), _ptr(v_new),
        _ptr(kidx_new), _ptr(Kq), _ptr(Ksc), _ptr(Vq), _ptr(Vsc), _ptr(K_idx), _ptr(q_idx),
        _ptr(q), _ptr(gate), _ptr(ids), _ptr(n_sel), _ptr(out), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)), "qsa_step")


class StepCall:
    """One prepared qsa_step call: the descriptors and raw device pointers
    are marshalled once, so each call() is a single C call with no per-call
    Python work beyond it (for timing loops)."""

    def __init__(self, pdesc, idesc, adesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx,
                 q_idx, q, gate, ids, n_sel, out, ws, stream=None):
        _check_step(pdesc, idesc, adesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx, q_idx,
                    q, gate, ids, n_sel, out, ws, qsa_step_workspace(idesc, adesc))
        self._keep = (pdesc, idesc, adesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx,
                      q_idx, q, gate, ids, n_sel, out, ws)
        self._args = (ctypes.byref(pdesc), ctypes.byref(idesc), ctypes.byref(adesc),
                      _ptr(k_new), _ptr(v_new), _ptr(kidx_new), _ptr(Kq), _ptr(Ksc), _ptr(Vq),
                      _ptr(Vsc), _ptr(K_idx), _ptr(q_idx), _ptr(q), _ptr(gate), _ptr(ids),
                      _ptr(n_sel), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                      _stream(stream))
        self._fn = lib().qsa_step

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != 0:
            _check(rc, "qsa_step")


# ------------------------------------------------------- whole-path plan ---

class QsaPath:
    """Device buffers for one workload shape plus the three calls in order.

    Holds only torch-allocated device memory (inputs are passed in already on
    the GPU); run() enqueues index_topk -> attend -> merge on one stream.
    """

    def __init__(self, *, batch, T, N, di, k, pos0, dense_max, cap, Hq, Hkv, D, P,
                 q_f16=False, out_f16=False, scale=None, device="cuda", strides=None,
                 algo=QSA_ATTEND_AUTO):
        self.idesc = index_desc(batch=batch, T=T, n_cells=N, d_idx=di, k=k, pos0=pos0,
                                dense_max=dense_max, ids_cap=cap)
        self.adesc = attn_desc(batch=batch, T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, ids_cap=cap,
                               n_cells=N, scale=scale,
                               q_dtype=QSA_F16 if q_f16 else QSA_F32,
                               out_dtype=QSA_F16 if out_f16 else QSA_F32, strides=strides,
                               algo=algo)
        ws_bytes = qsa_index_topk_workspace(self.idesc)
        n_part = qsa_partials_floats(self.adesc)
        if ws_bytes == 0 or n_part == 0:
            raise QsaError("unsupported or invalid workload shape")
        self.ws = torch.empty(ws_bytes // 4, dtype=torch.int32, device=device)
        self.ids = torch.empty((batch, T, cap), dtype=torch.int32, device=device)
        self.n_sel = torch.empty((batch, T), dtype=torch.int32, device=device)
        self.partials = torch.empty(n_part, dtype=torch.float32, device=device)
        self.out = torch.empty((batch, T, Hq, D),
                               dtype=torch.float16 if out_f16 else torch.float32,
                               device=device)
        rows = batch * T * Hq * P
        self.pm = self.partials[:rows].view(batch, T, Hq, P)
        self.pl = self.partials[rows:2 * rows].view(batch, T, Hq, P)
        self.po = self.partials[2 * rows:].view(batch, T, Hq, P, D)

    def index(self, q_idx, K_idx, stream=None):
        qsa_index_topk(self.idesc, q_idx, K_idx, self.ids, self.n_sel, self.ws, stream)

    def attend(self, q, Kq, Ksc, Vq, Vsc, stream=None, ids=None, n_sel=None):
        qsa_attend(self.adesc, q, Kq, Ksc, Vq, Vsc, self.ids if ids is None else ids,
                   self.n_sel if n_sel is None else n_sel, self.partials, stream)

    def merge(self, stream=None, gate=None):
        if gate is None:
            qsa_merge(self.adesc, self.partials, self.out, stream)
        else:
            qsa_merge_gated(self.adesc, self.partials, gate, self.out, stream)

    def attend_merge(self, q, Kq, Ksc, Vq, Vsc, stream=None, gate=None, ids=None,
                     n_sel=None):
        qsa_attend_merge(self.adesc, q, Kq, Ksc, Vq, Vsc, self.ids if ids is None else ids,
                         self.n_sel if n_sel is None else n_sel, gate, self.out, stream)

    def run(self, dev: dict, stream=None):
        self.index(dev["q_idx"], dev["K_idx"], stream)
        self.attend(dev["q"], dev["Kq"], dev["Ksc"], dev["Vq"], dev["Vsc"], stream)
        self.merge(stream, gate=dev.get("gate"))
        return self.out


def to_device(inp: dict, device="cuda") -> dict:
    """Copy the array fields of an input dict (numpy) to device tensors."""
    out = {}
    for key in ("q_idx", "K_idx", "q", "Kq", "Ksc", "Vq", "Vsc"):
        out[key] = torch.from_numpy(inp[key]).to(device)
    return out


def path_for(inp: dict, *, P: int | None = None, device="cuda", strides=None,
             algo: int = QSA_ATTEND_AUTO) -> QsaPath:
    """A QsaPath sized for an input dict produced by the seeded generator."""
    return QsaPath(batch=inp["batch"], T=inp["T"], N=inp["N"], di=inp["di"], k=inp["k"],
                   pos0=inp["pos0"], dense_max=inp["dense_max"], cap=inp["cap"],
                   Hq=inp["Hq"], Hkv=inp["Hkv"], D=inp["D"],
                   P=inp["P"] if P is None else P, q_f16=inp["q_dtype"] == "f16",
                   out_f16=inp["out_dtype"] == "f16", device=device, strides=strides,
                   algo=algo)
