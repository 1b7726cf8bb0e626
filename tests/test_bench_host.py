"""Host-side logic of bench.py (CPU): the single-GPU guard and the
algorithmic byte accounting that the HBM fractions and the roofline are
computed from."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _decode(**over):
    p = dict(T=1, N=8192, di=128, Hq=24, Hkv=2, D=256, k=2048, dense_max=2051, pos0=8191,
             q_dtype="f32", out_dtype="f32")
    p.update(over)
    return p


def test_decode_step_bytes_by_hand():
    """One decode problem keeping 2048 cells, counted term by term."""
    by = bench.algorithmic_bytes(_decode(), B=1, n_sel_total=2048)
    # new token: fp32 K and V rows and index key in; int8 codes, fp16 scales
    # and the fp16 index key out
    assert by["append"] == 2 * 2 * 256 * 4 + 128 * 4 + 2 * 2 * (256 + 8 * 2) + 128 * 2
    # every visible cell's fp16 index key once, plus the token's query
    assert by["index"] == 8192 * 256 + 256
    # per kept cell: K and V codes (256 B per head) and scales (16 B per
    # head), both heads, plus its 4-byte id; the fp32 query of 24 heads
    assert by["attend"] == 2048 * (2 * 2 * (256 + 16) + 4) + 24 * 256 * 4
    # the output and the gate, fp32
    assert by["out"] == 24 * 256 * 8
    assert by["total"] == by["append"] + by["index"] + by["attend"] + by["out"]


def test_dense_rows_read_no_index_keys():
    """A token that keeps every visible cell (dense fallback) never scans."""
    by = bench.algorithmic_bytes(_decode(pos0=2000), B=3, n_sel_total=3 * 2001)
    assert by["index"] == 0


def test_bytes_scale_with_the_batch():
    a = bench.algorithmic_bytes(_decode(), B=1, n_sel_total=2048)
    b = bench.algorithmic_bytes(_decode(), B=512, n_sel_total=512 * 2048)
    for key in a:
        assert b[key] == 512 * a[key]


def test_fp16_prompt_halves_query_output_and_gate_bytes():
    f32 = bench.algorithmic_bytes(_decode(), B=1, n_sel_total=2048)
    f16 = bench.algorithmic_bytes(_decode(q_dtype="f16", out_dtype="f16"), B=1,
                                  n_sel_total=2048)
    assert f32["out"] == 2 * f16["out"]
    assert f32["attend"] - f16["attend"] == 24 * 256 * 2
