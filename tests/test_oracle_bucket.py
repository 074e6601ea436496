"""Pins of the oracle's relative-distance bucket (CPU)."""
import numpy as np
import pytest

from oracle.bucket import bucket
from tests.oracle_pins_util import bucket_by_boundaries


@pytest.mark.parametrize("d,expect", [(0, 0), (1, 1), (15, 15), (16, 16), (19, 16), (20, 17), (31, 19),
                                      (32, 20), (4095, 47), (4096, 48), (32767, 59), (65535, 63),
                                      (10 ** 9, 63)])
def test_spot_values(d, expect):
    assert int(bucket(d)) == expect
    assert int(bucket(-d)) == expect


def test_exhaustive_against_boundary_enumeration():
    d = np.arange(-70000, 70000)
    np.testing.assert_array_equal(bucket(d), bucket_by_boundaries(d))


def test_monotone_and_range():
    b = bucket(np.arange(0, 70000))
    assert np.all(np.diff(b) >= 0)
    assert b.min() == 0 and b.max() == 63
    # every bucket is reached, buckets 60..63 only from distance 32768 on
    assert set(np.unique(b)) == set(range(64))
    assert bucket(np.arange(0, 32768)).max() == 59
