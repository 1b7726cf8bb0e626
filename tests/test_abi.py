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
