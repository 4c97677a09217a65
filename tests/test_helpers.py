"""The error metrics used by the parity tests behave as documented."""
import numpy as np

from tests.helpers import slice_rel_err, state_rel_err


def test_slice_rel_err_is_per_slice():
    ref = np.zeros((2, 3, 4))
    ref[0] = 1.0
    ref[1] = 100.0
    got = ref.copy()
    got[0, 0, 0] += 0.01
    got[1, 0, 0] += 0.5
    assert abs(slice_rel_err(got, ref, 1) - 0.01) < 1e-12


def test_state_rel_err_floor():
    ref = np.zeros((1, 3, 2, 2))
    ref[0, 0] = 1.0
    ref[0, 1] = 1e-80          # decayed far below fp32 range
    got = ref.copy()
    got[0, 1] = 0.0            # fp32 flushes it
    assert state_rel_err(got, ref) < 1e-40
    got[0, 0, 0, 0] = 1.5
    assert abs(state_rel_err(got, ref) - 0.5) < 1e-12
    got = ref.copy()
    got[0, 2, 1, 1] = 1e-3     # a dead level that should be zero
    assert state_rel_err(got, ref) >= 1e3


def test_state_rel_err_floor_is_near_fp32_range():
    """A level 1e-12 of its pair's largest is held to the full tolerance: a
    20% error there must not pass as it did under a 1e-6 floor."""
    ref = np.zeros((1, 2, 2, 2))
    ref[0, 0] = 1.0
    ref[0, 1] = 1e-12
    got = ref.copy()
    got[0, 1] *= 1.2
    assert abs(state_rel_err(got, ref) - 0.2) < 1e-9
