"""Sensitivity of the oracle's pins: plant one plausible mistake at a time in a
copy of the oracle source (on the CPU), build it, and require that at least
one pin fails.  Each mutant runs in its own subprocess, so a mutant that
crashes counts as caught without taking the test run down."""
import os
import subprocess
import sys
import textwrap

import pytest

from oracle.oracle import SRC, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, exact source snippet, replacement)
MUTANTS = [
    ("tie_to_higher_index",
     "return (a->j < b->j) ? -1 : (a->j > b->j);",
     "return (a->j > b->j) ? -1 : (a->j < b->j);"),
    ("own_cell_invisible",
     "const int nvis = pos + 1;            /* cells 0..pos inclusive */",
     "const int nvis = pos > 0 ? pos : 1;"),
    ("dense_bound_off_by_one",
     "if (nvis <= dense_max) {",
     "if (nvis < dense_max) {"),
    ("gqa_interleaved",
     "const int g = h / G;",
     "const int g = h % Hkv;"),
    ("scale_block_index",
     "scales[row * (D / 32) + d / 32]",
     "scales[row * (D / 32) + d % (D / 32)]"),
    ("softmax_scale_dropped",
     "x[i] = scale * dot;",
     "x[i] = dot;"),
    ("chunk_len_floor",
     "const int S = (ns + P - 1) / P;",
     "const int S = (ns / P > 0) ? ns / P : 1;"),
    ("merge_l_unweighted",
     "L += l[c] * e;",
     "L += l[c];"),
    ("merge_exp_sign",
     "const double e = exp(m[c] - M);",
     "const double e = exp(M - m[c]);"),
    ("score_key_reversed",
     "s += qo_half_to_double(qt[i]) * qo_half_to_double(kj[i]);",
     "s += qo_half_to_double(qt[i]) * qo_half_to_double(kj[di - 1 - i]);"),
    ("ids_in_rank_order",
     "qsort(kept, (size_t)n, sizeof(int), qo_cmp_int);",
     "(void)qo_cmp_int;"),
    ("half_subnormal_scale",
     "v = ldexp((double)frac, -24);",
     "v = ldexp((double)frac, -25);"),
    ("half_round_half_up",
     "double r = nearbyint(ldexp(a, 10 - E));",
     "double r = floor(ldexp(a, 10 - E) + 0.5);"),
    ("exp_argument_sign",
     "const double p = exp(x[i] - m);",
     "const double p = exp(m - x[i]);"),
    ("v_reads_k",
     "oc[d] += p * qo_deq(Vq, Vsc, Hkv, D, j, g, d);",
     "oc[d] += p * qo_deq(Kq, Ksc, Hkv, D, j, g, d);"),
    ("f16_q_raw_bits",
     "qd[d] = q_is_f16 ? qo_half_to_double(((const uint16_t*)q)[qi])",
     "qd[d] = q_is_f16 ? (double)(((const uint16_t*)q)[qi])"),
    ("pad_with_zero",
     "row[r] = (r < n) ? kept[r] : -1;",
     "row[r] = (r < n) ? kept[r] : 0;"),
    ("k_not_clamped",
     "n = (k < nvis) ? k : nvis;",
     "n = k;"),
    ("quant_scale_over_128",
     "uint16_t h = qo_double_to_half(a / 127.0);",
     "uint16_t h = qo_double_to_half(a / 128.0);"),
    ("quant_ties_to_odd",
     "(err == best_err && fmod(fabs(c), 2.0) == 0.0)",
     "(err == best_err && fmod(fabs(c), 2.0) == 1.0)"),
    ("quant_no_clamp",
     "if (best > 127.0)\n        best = 127.0;",
     "if (best > 128.0)\n        best = 127.0;"),
    ("quant_absmax_first_element",
     "if (fabs((double)xb[e]) > a)",
     "if (e == 0)"),
    ("append_index_key_truncated",
     "K_idx[cell * di + i] = qo_double_to_half((double)kidx_new[(size_t)t * di + i]);",
     "K_idx[cell * di + i] = qo_double_to_half(trunc(ldexp((double)kidx_new[(size_t)t * di + i], 8)) / 256.0);"),
    ("append_wrong_cell",
     "const size_t cell = (size_t)(pos0 + t);",
     "const size_t cell = (size_t)(pos0 + t + 1 < N ? pos0 + t + 1 : pos0 + t);"),
    ("gate_sign",
     "out[i] *= 1.0 / (1.0 + exp(-gate[i]));",
     "out[i] *= 1.0 / (1.0 + exp(gate[i]));"),
    ("gate_tanh",
     "out[i] *= 1.0 / (1.0 + exp(-gate[i]));",
     "out[i] *= 0.5 * (1.0 + tanh(gate[i]));"),
    ("max_not_subtracted_last_chunk_only",
     "for (int c = 0; c < P; ++c)\n            if (m[c] > M)",
     "for (int c = 0; c + 1 < P; ++c)\n            if (m[c] > M)"),
]

RUNNER = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    from oracle.oracle import Oracle
    from tests.oracle_pins import ALL_PINS
    orc = Oracle({lib!r})
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # AssertionError or a rejected call
            failed.append(pin.__name__)
    print("FAILED:" + ",".join(failed))
    sys.exit(1 if failed else 0)
""")


def test_mutant_snippets_exist_once():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    build(str(msrc), lib)
    code = RUNNER.format(root=ROOT, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}{r.stderr}"
