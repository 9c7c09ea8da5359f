"""Pins of the oracle's Philox generator and its uniform mapping (CPU only)."""

import os

import numpy as np
import pytest
from scipy import stats

from oracle.philox import philox4, philox4x32, seed_key, uniform24

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((tuple(w[0:4]), tuple(w[4:6]), tuple(w[6:10])))
    return rows


def test_kat_file_present():
    assert len(_kat_rows()) == 3


@pytest.mark.parametrize("row", _kat_rows())
def test_philox4x32_10_known_answers(row):
    ctr, key, out = row
    assert philox4(ctr, key, width=32, rounds=10) == out


@pytest.mark.parametrize("row", _kat_rows())
def test_vectorised_matches_known_answers(row):
    ctr, key, out = row
    got = philox4x32(*ctr, *key)
    assert tuple(int(x) for x in got) == out


def test_width_generic_form_matches_numpy_philox4x64():
    """numpy's Philox bit generator is Philox4x64-10; it increments its counter before each block."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        ctr = [int(x) for x in rng.integers(0, 2**63, size=4)]
        key = [int(x) for x in rng.integers(0, 2**63, size=2)]
        bg = np.random.Philox(counter=ctr, key=key)
        raw = [int(x) for x in bg.random_raw(4)]
        nxt = list(ctr)
        nxt[0] += 1          # no carry: ctr[0] < 2**63
        assert philox4(nxt, key, width=64, rounds=10) == tuple(raw)


def test_vectorised_equals_scalar_on_random_counters():
    rng = np.random.default_rng(11)
    c = rng.integers(0, 2**32, size=(4, 257), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9ABCDEF0
    vec = philox4x32(c[0], c[1], c[2], c[3], k0, k1)
    for j in range(c.shape[1]):
        ref = philox4((c[0, j], c[1, j], c[2, j], c[3, j]), (k0, k1))
        assert tuple(int(v[j]) for v in vec) == ref


def test_seed_key_split():
    assert seed_key(0x0123456789ABCDEF) == (0x89ABCDEF, 0x01234567)


def test_uniform24_range_and_fp32_exactness():
    w = np.array([0, 1, 511, 512, 2**31, 2**32 - 1], dtype=np.uint64)
    u = uniform24(w)
    assert np.all(u > 0) and np.all(u < 1)
    assert u[0] == 2.0 ** -24 and u[-1] == 1.0 - 2.0 ** -24
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)


def test_uniformity_chi_square():
    n = 200_000
    idx = np.arange(n, dtype=np.uint64)
    u = uniform24(philox4x32(idx, 3, 5, 7, 0xDEADBEEF, 0x5EED)[1])
    counts, _ = np.histogram(u, bins=64, range=(0.0, 1.0))
    p = stats.chisquare(counts).pvalue
    assert p > 1e-4
