"""Pins for the oracle's Philox4x32-10: published known answers + uniformity."""
import os

import numpy as np
from scipy import stats

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat_rows():
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        w = [int(x, 16) for x in line.split()]
        yield w[:4], w[4:6], w[6:10]


def test_known_answer_vectors():
    rows = list(_kat_rows())
    assert len(rows) == 3
    for ctr, key, want in rows:
        got = philox.philox4x32(*ctr, *key)
        assert [int(x) for x in got] == want


def test_vectorised_matches_scalar():
    c = np.arange(1000)
    o = philox.philox4x32(c, 7, 3, 1, 0x1234, 0x5678)
    for i in (0, 17, 999):
        s = philox.philox4x32(i, 7, 3, 1, 0x1234, 0x5678)
        assert all(int(a[i]) == int(b) for a, b in zip(o, s))


def test_uniform_range_and_chisquare():
    u = philox.uniform(99, 3, 5, np.arange(1 << 20), philox.PURPOSE_DRAFT)
    assert u.min() >= 0.0 and u.max() < 1.0
    # exact 24-bit grid
    assert np.all(u * (1 << 24) == np.floor(u * (1 << 24)))
    counts = np.bincount((u * 256).astype(np.int64), minlength=256)
    chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
    assert stats.chi2.sf(chi2, 255) > 1e-3


def test_streams_differ_by_purpose_slot_step():
    a = philox.uniform(1, 0, 0, np.arange(64), 0)
    assert not np.array_equal(a, philox.uniform(1, 0, 0, np.arange(64), 1))
    assert not np.array_equal(a, philox.uniform(1, 1, 0, np.arange(64), 0))
    assert not np.array_equal(a, philox.uniform(1, 0, 1, np.arange(64), 0))
    assert not np.array_equal(a, philox.uniform(2, 0, 0, np.arange(64), 0))
    # the seed's high word is part of the key
    assert not np.array_equal(a, philox.uniform(1 + (1 << 32), 0, 0, np.arange(64), 0))
