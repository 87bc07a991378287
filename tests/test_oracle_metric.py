"""Pins for the layer-output parity measure, oracle.layer.rms and
max_err_over_rms: max over the whole [T][H] tensor of |got - ref|, divided by
the root mean square of every element of ref.  Values worked by hand, chosen
so that a mean in place of the max, a missing square root, a per-row RMS, a
signed (not absolute) error or an RMS of `got` instead of `ref` each give a
different number."""
import math

import numpy as np

from oracle import layer


def test_rms_by_hand():
    assert layer.rms([3.0, 4.0]) == math.sqrt(12.5)            # (9 + 16) / 2
    assert layer.rms([[1.0, 1.0], [3.0, 3.0]]) == math.sqrt(5.0)   # (1 + 1 + 9 + 9) / 4, one RMS for the tensor
    assert layer.rms([-2.0, 2.0, -2.0, 2.0]) == 2.0
    assert layer.rms(np.zeros(3)) == 0.0


def test_max_error_over_rms_by_hand():
    ref = np.array([[1.0, -1.0], [1.0, -1.0]])                 # RMS 1
    got = ref + np.array([[0.0, 0.5], [-2.0, 0.0]])
    # max |err| = 2 (a negative error), not the mean 0.625 nor the signed max 0.5
    assert layer.max_err_over_rms(got, ref) == 2.0
    ref = np.array([3.0, 4.0])                                  # RMS sqrt(12.5)
    got = np.array([3.0, 5.0])
    assert math.isclose(layer.max_err_over_rms(got, ref), 1.0 / math.sqrt(12.5), rel_tol=0, abs_tol=1e-15)
    # the denominator is the reference's RMS, not the result's
    ref = np.array([[1.0, 1.0], [3.0, 3.0]])                    # RMS sqrt(5)
    got = np.array([[1.0, 1.0], [3.0, 13.0]])                   # its own RMS is far larger
    assert math.isclose(layer.max_err_over_rms(got, ref), 10.0 / math.sqrt(5.0), rel_tol=0, abs_tol=1e-14)


def test_identical_outputs_have_zero_error_and_scale_invariance():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((3, 8))
    assert layer.max_err_over_rms(ref.copy(), ref) == 0.0
    got = ref + 1e-3 * rng.standard_normal((3, 8))
    a = layer.max_err_over_rms(got, ref)
    # scaling both tensors by a power of two leaves the measure unchanged, exactly
    assert layer.max_err_over_rms(8.0 * got, 8.0 * ref) == a
