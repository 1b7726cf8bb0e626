"""The pages' two bit-exact claims about the attention softmax, checked on the
CPU in fp32 and fp64 (r20 audit page, section 2 'qsa.metal'):

* holding two cells per lane and taking the max over lanes of each lane's
  max(s0, s1) gives exactly the max over all cells;
* adding a p1 = 0 term for an absent cell does not change the sum bit for bit.

The GPU tests re-check the same two properties on the HIP kernels (the
padding test and the per-chunk max against the oracle)."""
import numpy as np
import pytest


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("width", [32, 64])
def test_max_of_lane_maxima_is_exact(dtype, width):
    rng = np.random.default_rng(1)
    for n in (1, 5, width - 1, width, width + 1, 2 * width - 1, 2 * width):
        s = (rng.standard_normal(n) * 7).astype(dtype)
        lanes = np.full(2 * width, -np.inf, dtype=dtype)
        lanes[:n] = s
        s0, s1 = lanes[:width], lanes[width:]      # cells lane and lane+width
        per_lane = np.maximum(s0, s1)
        assert per_lane.max().tobytes() == s.max().tobytes()


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_zero_padding_keeps_sum_bitwise(dtype):
    rng = np.random.default_rng(2)
    for n in (1, 2, 3, 31, 33, 63):
        p = np.exp(rng.standard_normal(n)).astype(dtype)
        acc = dtype(0)
        for v in p:
            acc = dtype(acc + v)
        acc_pad = dtype(0)
        for v in p:
            acc_pad = dtype(acc_pad + v)
            acc_pad = dtype(acc_pad + dtype(0.0))  # absent partner cell, p1 = 0
        assert acc.tobytes() == acc_pad.tobytes()
