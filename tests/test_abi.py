"""The C ABI without a GPU: the library loads, exports every function that
include/qsa.h declares, the ctypes descriptors match the C struct layout, and
invalid calls are rejected on the host with the documented status codes
(nothing is launched, so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import top_sparse_attention_score_amd as qsa
from top_sparse_attention_score_amd import qsa as qb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"QSA_API\s+[\w\s\*]+?\b(qsa_\w+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("qsa_index_topk", "qsa_attend", "qsa_merge", "qsa_index_topk_workspace",
              "qsa_partials_floats", "qsa_status_string", "qsa_version", "qsa_kv_append",
              "qsa_merge_gated"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = qb.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", qb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared_functions()) <= exported
    # nothing but the C ABI is exported from the text segment
    assert exported == set(declared_functions()), exported - set(declared_functions())


def test_version_and_status_strings():
    assert qb.lib().qsa_version() == 1
    assert qb.status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert qb.status_string(code) not in ("ok", "unknown status")


def test_struct_layout_matches_c(tmp_path):
    fields_i = [f[0] for f in qb.IndexDesc._fields_]
    fields_a = [f[0] for f in qb.AttnDesc._fields_]
    fields_p = [f[0] for f in qb.AppendDesc._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "qsa.h"', "int main(void){",
           'printf("%zu %zu %zu\\n", sizeof(qsa_index_desc), sizeof(qsa_attn_desc), '
           'sizeof(qsa_append_desc));']
    src += [f'printf("%zu\\n", offsetof(qsa_index_desc, {f}));' for f in fields_i]
    src += [f'printf("%zu\\n", offsetof(qsa_attn_desc, {f}));' for f in fields_a]
    src += [f'printf("%zu\\n", offsetof(qsa_append_desc, {f}));' for f in fields_p]
    src += ["return 0;}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)],
                   check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(qb.IndexDesc)
    assert vals[1] == ctypes.sizeof(qb.AttnDesc)
    assert vals[2] == ctypes.sizeof(qb.AppendDesc)
    offs = vals[3:]
    exp = [getattr(qb.IndexDesc, f).offset for f in fields_i] + \
          [getattr(qb.AttnDesc, f).offset for f in fields_a] + \
          [getattr(qb.AppendDesc, f).offset for f in fields_p]
    assert offs == exp


def _idesc(**kw):
    base = dict(batch=1, T=1, n_cells=8192, d_idx=128, k=2048, pos0=8191, dense_max=2051,
                ids_cap=2051)
    base.update(kw)
    return qsa.index_desc(**base)


def _adesc(**kw):
    base = dict(batch=1, T=1, Hq=24, Hkv=2, D=256, P=32, ids_cap=2051, n_cells=8192)
    base.update(kw)
    strides = base.pop("strides", None)
    return qsa.attn_desc(strides=strides, **base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), INVALID), (dict(T=0), INVALID), (dict(k=0), INVALID),
    (dict(pos0=-1), INVALID), (dict(pos0=8192), INVALID), (dict(k=3000), INVALID),
    (dict(dense_max=3000), INVALID), (dict(d_idx=96), UNSUPPORTED),
    (dict(batch=70000), UNSUPPORTED),
])
def test_index_desc_rejected(kw, code):
    d = _idesc(**kw)
    assert qb.lib().qsa_index_topk_workspace(ctypes.byref(d)) == 0
    rc = qb.lib().qsa_index_topk(ctypes.byref(d), 16, 16, 16, 16, 16, 1 << 30, None)
    assert rc == code


def test_index_pointer_and_workspace_checks():
    d = _idesc()
    need = qb.lib().qsa_index_topk_workspace(ctypes.byref(d))
    assert need >= 8192 * 4          # at least one score key per visible cell
    L = qb.lib()
    assert L.qsa_index_topk(ctypes.byref(d), None, 16, 16, 16, 16, need, None) == INVALID
    assert L.qsa_index_topk(ctypes.byref(d), 8, 16, 16, 16, 16, need, None) == INVALID
    assert L.qsa_index_topk(ctypes.byref(d), 16, 16, 16, 16, None, need, None) == WORKSPACE
    assert L.qsa_index_topk(ctypes.byref(d), 16, 16, 16, 16, 16, need - 1, None) == WORKSPACE
    assert L.qsa_index_topk(ctypes.byref(d), 16, 16, 16, 16, 8, need, None) == WORKSPACE


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), INVALID), (dict(Hq=25), INVALID), (dict(D=48), INVALID),
    (dict(P=0), INVALID), (dict(P=65), UNSUPPORTED), (dict(D=128), UNSUPPORTED),
    (dict(Hq=6, Hkv=2), UNSUPPORTED), (dict(Hq=40, Hkv=2), UNSUPPORTED),
    (dict(scale=float("nan")), INVALID), (dict(q_dtype=2), INVALID),
    (dict(strides=dict(kq_cell_stride=520)), INVALID),
    (dict(strides=dict(ksc_cell_stride=34)), INVALID),
    (dict(strides=dict(vq_batch_stride=8)), INVALID),
    (dict(strides=dict(kq_cell_stride=-16)), INVALID),
    (dict(algo=3), INVALID), (dict(algo=-1), INVALID),
])
def test_attn_desc_rejected(kw, code):
    d = _adesc(**kw)
    L = qb.lib()
    assert L.qsa_partials_floats(ctypes.byref(d)) == 0
    assert L.qsa_attend(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 16, 16, None) == code
    assert L.qsa_merge(ctypes.byref(d), 16, 16, None) == code


def test_attn_pointer_checks_and_sizes():
    d = _adesc()
    L = qb.lib()
    rows = 24 * 32
    assert L.qsa_partials_floats(ctypes.byref(d)) == 2 * rows + rows * 256
    assert L.qsa_attend(ctypes.byref(d), None, 16, 16, 16, 16, 16, 16, 16, None) == INVALID
    assert L.qsa_attend(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 16, 8, None) == INVALID
    assert L.qsa_merge(ctypes.byref(d), 16, None, None) == INVALID
    assert L.qsa_merge(ctypes.byref(d), 16, 4, None) == INVALID
    # interleaved layout strides are accepted by validation
    d2 = _adesc(strides=dict(kq_cell_stride=1088, ksc_cell_stride=1088,
                             vq_cell_stride=1088, vsc_cell_stride=1088))
    assert L.qsa_partials_floats(ctypes.byref(d2)) > 0


def test_merge_gated_checks():
    L = qb.lib()
    d = _adesc()
    assert L.qsa_merge_gated(ctypes.byref(d), 16, 8, 16, None) == INVALID   # misaligned gate
    assert L.qsa_merge_gated(ctypes.byref(d), None, 16, 16, None) == INVALID
    assert L.qsa_merge_gated(None, 16, 16, 16, None) == INVALID
    assert L.qsa_merge_gated(ctypes.byref(_adesc(P=65)), 16, 16, 16, None) == UNSUPPORTED


def test_attend_merge_host_checks():
    """qsa_attend_merge validates like qsa_attend + qsa_merge_gated and
    rejects splits that one workgroup cannot merge, all before any launch."""
    L = qb.lib()
    d = _adesc(P=4)
    ins = [16] * 7                      # q, Kq, Ksc, Vq, Vsc, ids, n_sel
    args = ins + [16, 16]               # + gate, out
    assert L.qsa_attend_merge(None, *args, None) == INVALID
    assert L.qsa_attend_merge(ctypes.byref(d), None, *args[1:], None) == INVALID  # null q
    assert L.qsa_attend_merge(ctypes.byref(d), *ins, 16, None, None) == INVALID   # null out
    assert L.qsa_attend_merge(ctypes.byref(d), *ins, 16, 8, None) == INVALID      # misaligned out
    assert L.qsa_attend_merge(ctypes.byref(d), *ins, 8, 16, None) == INVALID      # misaligned gate
    for P in (3, 8, 16, 64):
        assert L.qsa_attend_merge(ctypes.byref(_adesc(P=P)), *args, None) == UNSUPPORTED
    assert L.qsa_attend_merge(ctypes.byref(_adesc(P=65)), *args, None) == UNSUPPORTED
    vec = _adesc(P=4)
    vec.algo = qb.QSA_ATTEND_VECTOR
    assert L.qsa_attend_merge(ctypes.byref(vec), *args, None) == UNSUPPORTED


def test_null_descriptor():
    L = qb.lib()
    assert L.qsa_index_topk(None, 16, 16, 16, 16, 16, 64, None) == INVALID
    assert L.qsa_attend(None, 16, 16, 16, 16, 16, 16, 16, 16, None) == INVALID
    assert L.qsa_merge(None, 16, 16, None) == INVALID


def _pdesc(**kw):
    base = dict(batch=2, T=1, n_cells=64, pos0=10, Hkv=2, D=256, d_idx=128)
    base.update(kw)
    strides = base.pop("strides", None)
    return qsa.append_desc(strides=strides, **base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), INVALID), (dict(T=0), INVALID), (dict(pos0=-1), INVALID),
    (dict(pos0=64), INVALID), (dict(T=3, pos0=62), INVALID), (dict(D=48), INVALID),
    (dict(D=2048), UNSUPPORTED), (dict(d_idx=6), INVALID), (dict(Hkv=0), INVALID),
    (dict(strides=dict(kq_cell_stride=520)), INVALID),
    (dict(strides=dict(vsc_cell_stride=33)), INVALID),
])
def test_append_desc_rejected(kw, code):
    d = _pdesc(**kw)
    L = qb.lib()
    assert L.qsa_kv_append(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 16, 16, None) == code


def test_append_pointer_checks():
    L = qb.lib()
    d = _pdesc()
    assert L.qsa_kv_append(ctypes.byref(d), None, 16, 16, 16, 16, 16, 16, 16, None) == INVALID
    assert L.qsa_kv_append(ctypes.byref(d), 8, 16, 16, 16, 16, 16, 16, 16, None) == INVALID
    assert L.qsa_kv_append(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 16, None, None) == INVALID
    assert L.qsa_kv_append(ctypes.byref(d), 16, 16, 16, 16, 1, 16, 16, 16, None) == INVALID
    d.reserved = 1
    assert L.qsa_kv_append(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 16, 16, None) == INVALID
    assert L.qsa_kv_append(None, 16, 16, 16, 16, 16, 16, 16, 16, None) == INVALID


def test_noalloc_index_host_checks():
    """qsa_index_topk_noalloc validates like qsa_index_topk and rejects a
    shape whose workspace exceeds its fixed array before touching the GPU."""
    L = qb.lib()
    assert L.qsa_index_topk_noalloc(None, 16, 16, 16, 16, None) == INVALID
    assert L.qsa_index_topk_noalloc(ctypes.byref(_idesc(batch=0)), 16, 16, 16, 16, None) == INVALID
    assert L.qsa_index_topk_noalloc(ctypes.byref(_idesc(d_idx=96)), 16, 16, 16, 16,
                                    None) == UNSUPPORTED
    assert L.qsa_index_topk_noalloc(ctypes.byref(_idesc()), None, 16, 16, 16, None) == INVALID
    big = _idesc(T=2048, n_cells=65536, pos0=63488)
    assert L.qsa_index_topk_workspace(ctypes.byref(big)) > qsa.QSA_NOALLOC_WORKSPACE_BYTES
    assert L.qsa_index_topk_noalloc(ctypes.byref(big), 16, 16, 16, 16, None) == WORKSPACE


def _window_call(pd, idsc, ad, ws=256, ws_bytes=1 << 30, kidx=16, gate=16):
    # 16 stands for any 16-byte aligned device pointer; nothing is launched
    # because every case below fails validation.
    return qb.lib().qsa_decode_window(
        None if pd is None else ctypes.byref(pd), None if idsc is None else ctypes.byref(idsc),
        None if ad is None else ctypes.byref(ad), 16, 16, kidx, 16, 16, 16, 16, 16, 16, 16,
        gate, 16, 16, 16, ws, ws_bytes, None)


def _window_descs(**kw):
    B, N, pos0 = kw.pop("batch", 2), kw.pop("n_cells", 8192), kw.pop("pos0", 8191)
    pd = _pdesc(batch=B, n_cells=N, pos0=pos0, Hkv=2, D=256, d_idx=128)
    idsc = _idesc(batch=B, n_cells=N, pos0=pos0)
    ad = _adesc(batch=B, n_cells=N)
    return pd, idsc, ad


def test_window_workspace_size():
    _, idsc, ad = _window_descs()
    L = qb.lib()
    need = L.qsa_decode_window_workspace(ctypes.byref(idsc), ctypes.byref(ad))
    rows = 2 * 24 * 32
    assert need >= 2 * 8192 * 4 + rows * (2 + 256) * 4
    assert L.qsa_decode_window_workspace(ctypes.byref(_idesc(batch=0)), ctypes.byref(ad)) == 0
    assert L.qsa_decode_window_workspace(ctypes.byref(idsc), ctypes.byref(_adesc(D=48))) == 0


def test_window_host_checks():
    """qsa_decode_window validates its three descriptors, their agreement and
    the workspace on the host; every rejected call enqueues nothing."""
    pd, idsc, ad = _window_descs()
    assert _window_call(None, idsc, ad) == INVALID
    assert _window_call(pd, None, ad) == INVALID
    assert _window_call(pd, idsc, None) == INVALID
    # descriptors that disagree
    for bad in (dict(T=2, pos0=8190), dict(pos0=100), dict(batch=3), dict(D=64),
                dict(Hkv=1), dict(n_cells=8000, pos0=7999)):
        p2 = _pdesc(**{**dict(batch=2, n_cells=8192, pos0=8191, Hkv=2, D=256, d_idx=128),
                       **bad})
        assert _window_call(p2, idsc, ad) == INVALID, bad
    assert _window_call(pd, _idesc(batch=2, n_cells=8192, pos0=8191, ids_cap=2100), ad) == INVALID
    assert _window_call(pd, idsc, _adesc(batch=2, n_cells=8192, T=2)) == INVALID
    assert _window_call(pd, idsc, _adesc(batch=2, n_cells=8192,
                                         strides=dict(kq_cell_stride=1024))) == INVALID
    # d_idx must agree only when a new index key is written
    p64 = _pdesc(batch=2, n_cells=8192, pos0=8191, Hkv=2, D=256, d_idx=64)
    assert _window_call(p64, idsc, ad) == INVALID
    # shapes and dtypes without a window kernel
    for kw in (dict(q_dtype=1), dict(out_dtype=1), dict(algo=2), dict(P=6), dict(P=2)):
        assert _window_call(pd, idsc, _adesc(batch=2, n_cells=8192, **kw)) == UNSUPPORTED, kw
    pl = _pdesc(batch=2, n_cells=20000, pos0=16384, Hkv=2, D=256, d_idx=128)
    assert _window_call(pl, _idesc(batch=2, n_cells=20000, pos0=16384),
                        _adesc(batch=2, n_cells=20000)) == UNSUPPORTED       # row too long
    pd8 = _pdesc(batch=2, n_cells=8192, pos0=8191, Hkv=3, D=256, d_idx=128)
    assert _window_call(pd8, idsc, _adesc(batch=2, n_cells=8192, Hkv=3)) == UNSUPPORTED
    # workspace
    need = qb.lib().qsa_decode_window_workspace(ctypes.byref(idsc), ctypes.byref(ad))
    assert _window_call(pd, idsc, ad, ws=None) == WORKSPACE
    assert _window_call(pd, idsc, ad, ws_bytes=need - 1) == WORKSPACE
    assert _window_call(pd, idsc, ad, ws=16) == WORKSPACE             # not 256-byte aligned
    # misaligned gate and output
    assert _window_call(pd, idsc, ad, gate=8) == INVALID


def _step_call(pd, idsc, ad, ws=256, ws_bytes=1 << 30, kidx=16, gate=16):
    # as _window_call: every case below fails validation, nothing launches
    return qb.lib().qsa_step(
        None if pd is None else ctypes.byref(pd), None if idsc is None else ctypes.byref(idsc),
        None if ad is None else ctypes.byref(ad), 16, 16, kidx, 16, 16, 16, 16, 16, 16, 16,
        gate, 16, 16, 16, ws, ws_bytes, None)


def test_step_workspace_size():
    """The index workspace, plus the partials only when the merge is not
    fused into the attention (P outside {1, 2, 4}, or the vector kernel)."""
    L = qb.lib()
    _, idsc, _ = _window_descs()
    iws = L.qsa_index_topk_workspace(ctypes.byref(idsc))
    fused = L.qsa_step_workspace(ctypes.byref(idsc), ctypes.byref(_adesc(batch=2, P=4)))
    split = L.qsa_step_workspace(ctypes.byref(idsc), ctypes.byref(_adesc(batch=2, P=8)))
    vec = L.qsa_step_workspace(ctypes.byref(idsc), ctypes.byref(_adesc(batch=2, P=4, algo=2)))
    assert iws <= fused < iws + 256
    rows = 2 * 24 * 8
    assert split >= fused + rows * (2 + 256) * 4
    assert vec >= fused + 2 * 24 * 4 * (2 + 256) * 4
    assert L.qsa_step_workspace(ctypes.byref(_idesc(batch=0)), ctypes.byref(_adesc())) == 0
    assert L.qsa_step_workspace(ctypes.byref(idsc), ctypes.byref(_adesc(D=48))) == 0


def test_step_host_checks():
    """qsa_step validates the three descriptors, their agreement and the
    workspace on the host; every rejected call enqueues nothing."""
    pd, idsc, ad = _window_descs()
    assert _step_call(None, idsc, ad) == INVALID
    assert _step_call(pd, None, ad) == INVALID
    assert _step_call(pd, idsc, None) == INVALID
    for bad in (dict(pos0=100), dict(batch=3), dict(D=64), dict(Hkv=1),
                dict(n_cells=8000, pos0=7999)):
        p2 = _pdesc(**{**dict(batch=2, n_cells=8192, pos0=8191, Hkv=2, D=256, d_idx=128),
                       **bad})
        assert _step_call(p2, idsc, ad) == INVALID, bad
    # T must agree across the three descriptors
    p2 = _pdesc(batch=2, T=2, n_cells=8192, pos0=8190, Hkv=2, D=256, d_idx=128)
    assert _step_call(p2, idsc, ad) == INVALID
    assert _step_call(pd, _idesc(batch=2, n_cells=8192, pos0=8191, ids_cap=2100), ad) == INVALID
    assert _step_call(pd, idsc, _adesc(batch=2, n_cells=8192, T=2)) == INVALID
    assert _step_call(pd, idsc, _adesc(batch=2, n_cells=8192,
                                       strides=dict(kq_cell_stride=1024))) == INVALID
    p64 = _pdesc(batch=2, n_cells=8192, pos0=8191, Hkv=2, D=256, d_idx=64)
    assert _step_call(p64, idsc, ad) == INVALID
    assert _step_call(pd, idsc, _adesc(batch=2, n_cells=8192, P=65)) == UNSUPPORTED
    need = qb.lib().qsa_step_workspace(ctypes.byref(idsc), ctypes.byref(ad))
    assert _step_call(pd, idsc, ad, ws=None) == WORKSPACE
    assert _step_call(pd, idsc, ad, ws_bytes=need - 1) == WORKSPACE
    assert _step_call(pd, idsc, ad, ws=16) == WORKSPACE               # not 256-byte aligned
    assert _step_call(pd, idsc, ad, gate=8) == INVALID


def test_probe_library_exports():
    """The bandwidth probe bench.py uses is its own library with exactly its
    three C entry points."""
    from top_sparse_attention_score_amd.build import PROBE_LIB
    assert os.path.exists(PROBE_LIB), "run __graft_entry__.build()"
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == {"hbm_probe_stream", "hbm_probe_gather", "hbm_probe_gather_sink_words"}
    L = ctypes.CDLL(PROBE_LIB)
    L.hbm_probe_gather_sink_words.restype = ctypes.c_longlong
    assert L.hbm_probe_gather_sink_words(256, 2, 4) == 512
    # invalid arguments are rejected before any launch
    L.hbm_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_void_p]
    assert L.hbm_probe_stream(None, 16, 16, 1, None) != 0
    assert L.hbm_probe_stream(16, 15, 16, 1, None) != 0
