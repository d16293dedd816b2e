"""The GPU tests' half-copy bound (tests/gpu_harness.py), on constructed values.

The half copy must be within 1 ulp of the oracle's, except where the master's own bound
(2e-6 relative to the terms of the update) spans more than that, as when an update
nearly cancels the weight: there any rounding of a master inside the master's bound is
accepted.  The GPU tests additionally require the half to equal the rounding of the
GPU's own stored master, bit for bit."""
import numpy as np
import pytest

import workloads as W
from gpu_harness import assert_half_close
from oracle import oracle as O


def _half(dtype, x):
    return O.float_to_half(dtype, np.asarray(x, np.float32))


@pytest.mark.parametrize("dtype", [W.F16, W.BF16], ids=["f16", "bf16"])
def test_one_ulp_where_the_master_bound_is_fine(dtype):
    w = np.array([0.25, -1.5, 3.0e-3], np.float32)
    want = _half(dtype, w)
    scale = np.abs(w).astype(np.float64)         # no cancellation: bound 2e-6 relative
    one_up = (want.astype(np.int32) + 1).astype(np.uint16)
    assert_half_close(one_up, want, "", dtype, w, scale)
    two_up = (want.astype(np.int32) + 2).astype(np.uint16)
    with pytest.raises(AssertionError):
        assert_half_close(two_up, want, "", dtype, w, scale)
    with pytest.raises(AssertionError):
        assert_half_close(two_up, want)           # the plain 1-ulp form


def test_near_cancellation_accepts_roundings_inside_the_master_bound():
    # bf16: a result of 3.2e-9 left by terms of size 1e-2: the master bound is
    # 2e-6 * 1e-2 = 2e-8, many bf16 ulps (1.5e-11) at 3.2e-9
    dtype = W.BF16
    w = np.array([3.2e-9], np.float32)
    want = _half(dtype, w)
    scale = np.array([1e-2])
    near = _half(dtype, w * (1 + 1e-2))                 # 3e-11 away: inside 2e-8
    assert abs(int(near[0]) - int(want[0])) >= 2
    assert_half_close(near, want, "", dtype, w, scale)
    far = _half(dtype, np.float32(3.2e-9 + 5e-8))      # 5e-8 away: outside
    with pytest.raises(AssertionError):
        assert_half_close(far, want, "", dtype, w, scale)
    sign = _half(dtype, -w)                             # wrong sign, well outside
    with pytest.raises(AssertionError):
        assert_half_close(sign, want, "", dtype, w, np.array([1e-12]))
