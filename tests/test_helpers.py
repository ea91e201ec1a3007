"""The parity check itself: one wrong row among thousands must fail it."""
import numpy as np
import pytest

from helpers import TOL, check_outputs, rel_l2, workloads_bf16


def test_row_check_catches_one_wrong_row():
    rng = np.random.default_rng(0)
    ref = rng.normal(size=(16384, 256))
    got = workloads_bf16(ref)                      # bf16 rounding: about 2e-3 per row
    check_outputs(got, ref, TOL["bf16"])
    for bad in ("zero", "scale", "swap"):
        g = got.copy()
        if bad == "zero":
            g[1234] = 0
        elif bad == "scale":
            g[1234] = workloads_bf16(1.05 * ref[1234])
        else:
            g[[10, 11]] = g[[11, 10]]
        # the whole-tensor norm alone lets each of these through
        assert rel_l2(g, ref) <= TOL["bf16"], bad
        with pytest.raises(AssertionError):
            check_outputs(g, ref, TOL["bf16"])


def test_row_check_catches_nan():
    ref = np.ones((8, 64))
    got = workloads_bf16(ref)
    got[3, 5] = 0x7FC0   # a bf16 NaN
    with pytest.raises(AssertionError):
        check_outputs(got, ref, TOL["bf16"])
