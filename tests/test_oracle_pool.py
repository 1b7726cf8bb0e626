"""The threaded, sliced oracle run used for the full prompt-chunk parity test
gives exactly what one oracle call over all tokens gives (tokens are
independent, so the slicing cannot change any result)."""
import math

import numpy as np

from datagen import make_inputs
from tests.oracle_pool import oracle_all_tokens


def test_sliced_oracle_equals_one_call(orc):
    inp = make_inputs("decode", seed=8900, batch=2, N=3000, T=7, pos0=2040, k=64,
                      dense_max=67, q_dtype="f16", out_dtype="f16")
    one = orc.run(inp, P=1, scale=1.0 / math.sqrt(inp["D"]))
    pool = oracle_all_tokens(orc, inp, P=1, scale=1.0 / math.sqrt(inp["D"]), slice_tokens=3,
                             threads=3)
    assert np.array_equal(pool["ids"], one["ids"])
    assert np.array_equal(pool["n_sel"], one["n_sel"])
    assert np.array_equal(pool["out"], one["out"])
