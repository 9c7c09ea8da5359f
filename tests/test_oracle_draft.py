"""Pins of the oracle's draft-step draw (CPU only).

The draw is pinned by its distribution (a chi-square test against softmax
over thousands of independent rows), by the Gumbel-max identity (the same
uniforms give the same winner through a different formula), by softmax's
shift invariance, by the limits (one finite logit, very sharp logits), and
by scipy's log_softmax for the returned log-probability.
"""

import numpy as np
import pytest
from scipy import special, stats

from oracle.draft import STREAM_DRAFT, draft_sample
from oracle.sample import uniforms


def test_distribution_matches_softmax_chi_square():
    V, B = 7, 4000
    l = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -3.0, 0.7])
    p = special.softmax(l)
    counts = np.zeros(V)
    for node in (1, 2, 3):
        r = draft_sample(np.tile(l, (B, 1)), seed=77, offset=5, node=node)
        counts += np.bincount(r["token"], minlength=V)
    chi2 = stats.chisquare(counts, counts.sum() * p)
    assert chi2.pvalue > 1e-3, chi2


def test_gumbel_max_identity():
    """argmax p/E and argmax l - ln(-ln U) are the same winner."""
    rng = np.random.default_rng(0)
    B, V = 20, 3001
    l = rng.standard_normal((B, V)) * 3
    seed, offset, node = 12345, 2, 4
    r = draft_sample(l, seed, offset, node)
    ids = np.arange(V)
    for b in range(B):
        u = uniforms(seed, ids // 4, node, b, 4 * offset + STREAM_DRAFT, ids % 4)
        assert r["token"][b] == int(np.argmax(l[b] - np.log(-np.log(u))))


def test_shift_invariance_and_logprob():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((6, 500)) * 2
    r1 = draft_sample(l, 9, 0, 1)
    r2 = draft_sample(l + 37.5, 9, 0, 1)
    assert np.array_equal(r1["token"], r2["token"])
    ref = special.log_softmax(l, axis=1)[np.arange(6), r1["token"]]
    np.testing.assert_allclose(r1["logprob"], ref, rtol=0, atol=1e-12)


def test_single_finite_logit_and_empty_rows():
    l = np.full((3, 40), -np.inf)
    l[0, 17] = 2.0
    l[1, 0] = -5.0
    r = draft_sample(l, 1, 0, 1)
    assert r["token"].tolist() == [17, 0, -1]
    assert r["logprob"][0] == 0.0 and r["logprob"][1] == 0.0 and np.isnan(r["logprob"][2])


def test_sharp_logits_pick_the_argmax():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((200, 1000)) * 1000.0
    r = draft_sample(l, 3, 0, 1)
    assert np.mean(r["token"] == np.argmax(l, axis=1)) >= 0.99


@pytest.mark.parametrize("what", ["node", "offset", "seed"])
def test_draws_differ_across_counters(what):
    l = np.zeros((64, 1000))
    base = dict(seed=5, offset=1, node=1)
    other = dict(base)
    other[what] += 1
    t1 = draft_sample(l, **base)["token"]
    t2 = draft_sample(l, **other)["token"]
    assert np.mean(t1 == t2) < 0.1
