"""Pins for ``oracle.compare``, the checker every parity test relies on (CPU
only).  Each expected value below is worked by hand in the comment beside it,
and each test is built so that a plausible slip in the checker (a wrong
denominator, a missing square root, a comparison turned around, an index
taken in the wrong order, a band sliced along the wrong axis) changes the
result."""
import math

import numpy as np
import pytest

from oracle import compare


def test_rel_l2_hand_values():
    # out - ref = (-1, 1): |d| = sqrt(2); |ref| = 2 -> sqrt(2) / 2.
    # Dividing by |out| = sqrt(2) would give 1; no square root would give 0.5.
    assert compare.rel_l2([1.0, 1.0], [2.0, 0.0]) == pytest.approx(math.sqrt(2.0) / 2.0, rel=1e-15)
    # 2-D arrays are one vector: d = (3, 0, 0, 4) -> 5; |ref| = sqrt(1+4+4+16) = 5 -> 1.
    out = np.array([[4.0, 2.0], [2.0, 8.0]])
    ref = np.array([[1.0, 2.0], [2.0, 4.0]])
    assert compare.rel_l2(out, ref) == pytest.approx(1.0, rel=1e-15)
    # argument order matters: |d| = 5 over |out| = sqrt(16+4+4+64) = sqrt(88)
    assert compare.rel_l2(ref, out) == pytest.approx(5.0 / math.sqrt(88.0), rel=1e-15)
    # a zero reference returns the absolute norm of the difference
    assert compare.rel_l2([3.0, 4.0], [0.0, 0.0]) == pytest.approx(5.0, rel=1e-15)
    assert compare.rel_l2([1.5, -2.0], [1.5, -2.0]) == 0.0


def test_rel_l2_sees_nan():
    assert math.isnan(compare.rel_l2([1.0, float("nan")], [1.0, 2.0]))


def test_first_mismatch_hand_values():
    ref = np.array([1.0, 2.0, 4.0])
    # bound atol + rtol |ref| = (0.5, 1, 2) with rtol 0.5: differences equal to
    # the bound pass (the comparison is <=)
    assert compare.first_mismatch([1.5, 2.0, 6.0], ref, rtol=0.5, atol=0.0) is None
    # 6.5 - 4 = 2.5 > 2: element 2 fails
    assert compare.first_mismatch([1.5, 2.0, 6.5], ref, rtol=0.5, atol=0.0) == ((2,), 6.5, 4.0)
    # below the reference fails the same way (absolute difference)
    assert compare.first_mismatch([1.0, 0.9, 4.0], ref, rtol=0.5, atol=0.0) == ((1,), 0.9, 2.0)
    # atol alone: |d| = 0.25 against 0.2 fails, against 0.25 passes
    assert compare.first_mismatch([1.25], [1.0], rtol=0.0, atol=0.2) == ((0,), 1.25, 1.0)
    assert compare.first_mismatch([1.25], [1.0], rtol=0.0, atol=0.25) is None


def test_first_mismatch_index_order_and_array_bound():
    ref = np.zeros((3, 4))
    out = ref.copy()
    out[2, 0] = 5.0
    out[1, 2] = 1.0
    # C order: (1, 2) comes before (2, 0)
    assert compare.first_mismatch(out, ref, rtol=0.0, atol=0.5) == ((1, 2), 1.0, 0.0)
    # a per-element bound: row 1 allows 2, so (1, 2) passes and (2, 0) fails
    bound = np.full((3, 4), 0.5)
    bound[1] = 2.0
    assert compare.first_mismatch(out, ref, rtol=0.0, atol=bound) == ((2, 0), 5.0, 0.0)
    assert compare.count_mismatch(out, ref, rtol=0.0, atol=bound) == 1
    assert compare.count_mismatch(out, ref, rtol=0.0, atol=0.5) == 2


def test_first_mismatch_counts_nan_and_inf():
    got = compare.first_mismatch([1.0, float("nan")], [1.0, 1.0], rtol=1.0, atol=1.0)
    assert got[0] == (1,) and math.isnan(got[1])
    assert compare.first_mismatch([float("inf")], [1.0], rtol=1.0, atol=1.0)[0] == (0,)
    assert compare.count_mismatch([float("nan"), 1.0], [1.0, float("nan")], rtol=1.0, atol=1.0) == 2


def test_band_report_hand_values():
    ref = np.ones((2, 10, 3))
    out = ref.copy()
    out[:, 8:, :] = 2.0   # only the last two positions along axis 1 are off
    head, tail = compare.band_report(out, ref, 4, axis=1)
    assert head == 0.0
    # tail band = positions 6..9: 2 of 4 positions off by 1 -> |d|^2 = 2*2*3 = 12,
    # |ref|^2 = 2*4*3 = 24 -> sqrt(1/2)
    assert tail == pytest.approx(math.sqrt(0.5), rel=1e-15)
    # along axis 0 both bands cover everything: sqrt(12 / 60)
    h0, t0 = compare.band_report(out, ref, 4, axis=0)
    assert h0 == pytest.approx(math.sqrt(12.0 / 60.0), rel=1e-15) and t0 == h0
    # along axis 2 (length 3) the bands are whole again
    assert compare.band_report(out, ref, 2, axis=2)[0] == pytest.approx(math.sqrt(8.0 / 40.0), rel=1e-15)


def test_band_errors_hand_values():
    ref = np.ones((1, 10))
    out = ref.copy()
    out[0, 5] = 3.0                       # one position of band 1 (positions 4..7)
    errs = compare.band_errors(out, ref, 4, axis=1)
    assert len(errs) == 3                 # 4 + 4 + 2
    assert errs[0] == 0.0 and errs[2] == 0.0
    assert errs[1] == pytest.approx(1.0, rel=1e-15)   # |d| = 2, |ref| = 2
    # the global norm hides it much better: 2 / sqrt(10)
    assert compare.rel_l2(out, ref) == pytest.approx(2.0 / math.sqrt(10.0), rel=1e-15)
