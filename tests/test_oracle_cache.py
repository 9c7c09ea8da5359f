"""Pins of the oracle's KV commit and draft-ring rewind (CPU only).

The commit is pinned by a hand-worked example (row labels written out by
hand), by the chain case (nothing moves), and by attention: after the commit
a plain causal pass over the compacted cache must give, for every accepted
node, the same output the candidate-tree mask gave that node before it.  The
rewind is pinned by hand-worked numbers and by a list simulation of the
draft's appended entries.
"""

import numpy as np
import pytest

from oracle.attention import ancestors, verify_attention
from oracle.cache import commit_path, rollback_draft
from oracle.sample import spec_sample
from workloads import chain_parent, make_attention_inputs, make_sample_inputs, random_tree


def _labelled_cache(B, Hkv, L_cap, D):
    """k[b,h,t,:] = 1000*b + 100*h + t, v = -k: every row says where it came from."""
    b = np.arange(B)[:, None, None, None]
    h = np.arange(Hkv)[None, :, None, None]
    t = np.arange(L_cap)[None, None, :, None]
    k = (1000 * b + 100 * h + t + np.zeros((1, 1, 1, D))).astype(np.float64)
    return k, -k


def test_hand_worked_example():
    # n_q = 5, kv_len = 7: block at positions 2..6, path nodes 0, 2, 3.
    k, v = _labelled_cache(1, 1, 8, 2)
    path = np.array([[0, 2, 3, -1, -1]])
    k2, v2, L2 = commit_path(k, v, [7], path, [3], n_q=5)
    assert L2.tolist() == [5]
    assert k2[0, 0, :, 0].tolist() == [0, 1, 2, 4, 5, 5, 6, 7]
    assert v2[0, 0, :, 1].tolist() == [0, -1, -2, -4, -5, -5, -6, -7]
    # The inputs are not modified.
    assert k[0, 0, :, 0].tolist() == list(range(8))


def test_hand_worked_two_sequences_two_heads():
    k, v = _labelled_cache(2, 2, 6, 1)
    path = np.array([[0, 1, 3, -1], [0, -1, -1, -1]])
    k2, _, L2 = commit_path(k, v, [6, 4], path, [3, 1], n_q=4)
    assert L2.tolist() == [5, 1]
    assert k2[0, 1, :, 0].tolist() == [100, 101, 102, 103, 105, 105]
    assert k2[1, 0, :, 0].tolist() == [1000, 1001, 1002, 1003, 1004, 1005]


def test_chain_changes_only_the_length():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((2, 3, 40, 8))
    v = rng.standard_normal((2, 3, 40, 8))
    n_q = 5
    counts = np.array([1, 5])
    path = np.tile(np.arange(n_q), (2, 1))
    path[0, 1:] = -1
    k2, v2, L2 = commit_path(k, v, [40, 23], path, counts, n_q)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    assert L2.tolist() == [36, 23]


def test_sampler_flagged_sequence_is_left_alone():
    k, v = _labelled_cache(1, 1, 6, 1)
    k2, v2, L2 = commit_path(k, v, [6], np.full((1, 3), -1), [0], n_q=3)
    assert np.array_equal(k2, k) and L2.tolist() == [6]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_committed_cache_reproduces_tree_attention(seed):
    """Causal attention over the compacted cache = tree-masked attention of the path nodes."""
    n_q, B, Hq, Hkv, D, L = 12, 2, 4, 2, 16, 50
    rng = np.random.default_rng(seed)
    parent = random_tree(n_q, seed=100 + seed)
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, L, dtype="f32", seed=seed)
    o_tree, _ = verify_attention(x["q"], x["k"], x["v"], x["kv_len"], parent=parent)
    q = x["q"].double().numpy()
    kv_len = x["kv_len"].numpy()
    paths = np.full((B, n_q), -1)
    counts = np.zeros(B, dtype=np.int64)
    for b in range(B):
        leaf = int(rng.integers(0, n_q))
        p = ancestors(parent, leaf)[::-1]          # root first
        paths[b, :len(p)] = p
        counts[b] = len(p)
    k2, v2, L2 = commit_path(x["k"].numpy(), x["v"].numpy(), kv_len, paths, counts, n_q)
    for b in range(B):
        c = int(counts[b])
        qb = q[b:b + 1, :, paths[b, :c]]           # the path nodes' queries, in path order
        o_chain, _ = verify_attention(qb, k2[b:b + 1], v2[b:b + 1], L2[b:b + 1])
        np.testing.assert_allclose(o_chain[0], o_tree[b][:, paths[b, :c]], rtol=0, atol=1e-12)


def test_sampler_path_commits():
    """spec_sample's path is a root-to-node chain of the tree and commits like one."""
    N, V = 16, 50
    parent = random_tree(N, seed=11)
    s = make_sample_inputs(3, N, V, parent, target_std=1.0, draft_noise_std=0.3, seed=5)
    r = spec_sample(s["target"], s["draft"], s["tokens"], parent, seed=9, offset=1)
    k, v = _labelled_cache(3, 1, N + 4, 1)
    k2, _, L2 = commit_path(k, v, [N + 4] * 3, r["out_path"], r["out_count"], n_q=N)
    for b in range(3):
        c = int(r["out_count"][b])
        p = r["out_path"][b, :c]
        assert p[0] == 0 and all(parent[p[j]] == p[j - 1] for j in range(1, c))
        assert L2[b] == 4 + c
        assert k2[b, 0, 4:4 + c, 0].tolist() == (1000 * b + 4 + p).tolist()


def test_rollback_hand_worked():
    # gamma = 4 chain: the draft appended nodes 0..3 (root + 3 fed-back drafts).
    total = np.array([100, 100, 100, 100])
    count = np.array([1, 2, 5, 0])
    assert rollback_draft(total, count, 4).tolist() == [97, 98, 100, 100]
    assert rollback_draft(total, count, 0).tolist() == [100, 100, 100, 100]


@pytest.mark.parametrize("gamma", [1, 3, 6])
def test_rollback_matches_list_simulation(gamma):
    """Keep a list of appended node ids, delete the rejected ones, compare lengths."""
    rng = np.random.default_rng(gamma)
    for _ in range(20):
        T0 = int(rng.integers(10, 50))
        appended = int(rng.integers(0, gamma + 1))
        count = int(rng.integers(1, gamma + 2))
        history = ["old"] * (T0 - appended) + [("node", j) for j in range(appended)]
        kept = [e for e in history if e == "old" or e[1] < count]
        assert rollback_draft([T0], [count], appended).tolist() == [len(kept)]


def test_chain_parent_path_is_identity():
    p = chain_parent(6)
    assert ancestors(p, 5)[::-1] == [0, 1, 2, 3, 4, 5]
