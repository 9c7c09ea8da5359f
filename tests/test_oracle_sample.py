"""Pins of the oracle's speculative-sampling tail (CPU only).

The sampler is random by nature, so it is pinned by the properties the pages
and the mathematics fix: acceptance probability = sum_x min(p_target, p_draft),
the closed-form count distribution (mean (1 - a^(g+1)) / (1 - a), "Speculative
Decoding & Medusa Architecture", section 1), the lossless property (every
emitted position follows the target distribution; "Speculative Decoding in
LLM Serving Systems", section "Accepting and rejecting"), the 1..gamma+1 bound,
and special cases with forced outcomes.
"""

import numpy as np
import pytest
import torch
from scipy import stats

from oracle.sample import race_draw, softmax, spec_sample
from workloads import chain_parent, make_sample_inputs, random_tree


def _rows(V, n, std, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(n, V, generator=g, dtype=torch.float32) * std


def _batch(rows, B):
    return rows[None].expand(B, -1, -1).contiguous()


def _chisq_ok(samples, probs, pmin=1e-3):
    V = probs.shape[0]
    counts = np.bincount(samples, minlength=V).astype(np.float64)
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    ex = ex * obs.sum() / ex.sum()
    return stats.chisquare(obs, ex).pvalue > pmin


def test_acceptance_probability_is_sum_of_min():
    V, B = 16, 20000
    t = _rows(V, 2, 1.5, 1)
    d = _rows(V, 2, 1.5, 2)
    x = make_sample_inputs(B, 2, V, None, 0, target=_batch(t, B), draft=_batch(d, B), seed=3)
    r = spec_sample(x["target"], x["draft"], x["tokens"], seed=77, offset=0)
    alpha = np.minimum(softmax(t[0].double().numpy()), softmax(d[0].double().numpy())).sum()
    rate = r["out_accept"][:, 1].mean()
    assert abs(rate - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / B)


def test_count_distribution_closed_form():
    """Identical rows at every position: P(count=k) = a^(k-1)(1-a) for k<=g, a^g for k=g+1."""
    V, B, gamma = 8, 20000, 3
    t = _rows(V, 1, 1.0, 5).repeat(gamma + 1, 1)
    d = _rows(V, 1, 1.0, 6).repeat(gamma + 1, 1)
    x = make_sample_inputs(B, gamma + 1, V, None, 0, target=_batch(t, B), draft=_batch(d, B),
                           seed=9)
    r = spec_sample(x["target"], x["draft"], x["tokens"], seed=1234, offset=5)
    a = np.minimum(softmax(t[0].double().numpy()), softmax(d[0].double().numpy())).sum()
    probs = np.array([a ** (k - 1) * (1 - a) for k in range(1, gamma + 1)] + [a ** gamma])
    counts = np.bincount(r["out_count"], minlength=gamma + 2)[1:]
    assert stats.chisquare(counts, probs * B).pvalue > 1e-3
    mean_closed = (1 - a ** (gamma + 1)) / (1 - a)
    sd = np.sqrt(np.sum(probs * np.arange(1, gamma + 2) ** 2) - mean_closed ** 2)
    assert abs(r["out_count"].mean() - mean_closed) < 4 * sd / np.sqrt(B)


def test_lossless_every_position_follows_the_target():
    V, B, gamma = 8, 24000, 3
    t = _rows(V, gamma + 1, 1.2, 11)
    d = _rows(V, gamma + 1, 1.2, 12)
    x = make_sample_inputs(B, gamma + 1, V, None, 0, target=_batch(t, B), draft=_batch(d, B),
                           seed=13)
    r = spec_sample(x["target"], x["draft"], x["tokens"], seed=99, offset=2)
    cnt, out = r["out_count"], r["out_tokens"]
    assert np.all((cnt >= 1) & (cnt <= gamma + 1))
    for pos in range(gamma + 1):
        sel = cnt >= pos + 1
        pt = softmax(t[pos].double().numpy())
        assert _chisq_ok(out[sel, pos], pt), f"position {pos}"


def test_equal_distributions_accept_everything():
    V, B, gamma = 32, 500, 4
    t = _rows(V, gamma + 1, 2.0, 21)
    x = make_sample_inputs(B, gamma + 1, V, None, 0, target=_batch(t, B), draft=_batch(t, B),
                           seed=22)
    r = spec_sample(x["target"], x["draft"], x["tokens"], seed=5)
    assert np.all(r["out_count"] == gamma + 1)
    assert np.array_equal(r["out_tokens"][:, :gamma], x["tokens"][:, 1:].numpy())


def test_disjoint_supports_reject_first_and_resample_target():
    V, B, gamma = 8, 6000, 3
    t = torch.full((gamma + 1, V), -np.inf)
    d = torch.full((gamma + 1, V), -np.inf)
    t[:, :4] = _rows(4, gamma + 1, 1.0, 31)
    d[:, 4:] = _rows(4, gamma + 1, 1.0, 32)
    x = make_sample_inputs(B, gamma + 1, V, None, 0, target=_batch(t, B), draft=_batch(d, B),
                           seed=33)
    r = spec_sample(x["target"], x["draft"], x["tokens"], seed=8)
    assert np.all(r["out_count"] == 1)
    assert np.all(r["residual"])
    assert _chisq_ok(r["out_tokens"][:, 0], softmax(t[0].double().numpy()))


def test_token_with_zero_target_mass_is_never_accepted():
    V, B = 8, 2000
    t = _rows(V, 2, 1.0, 41)
    t[0, 3] = -np.inf
    d = torch.full((2, V), -30.0)
    d[:, 3] = 0.0                         # the draft almost always proposes id 3
    x = make_sample_inputs(B, 2, V, None, 0, target=_batch(t, B), draft=_batch(d, B), seed=42)
    r = spec_sample(x["target"], x["draft"], x["tokens"], seed=3)
    prop3 = x["tokens"][:, 1].numpy() == 3
    assert prop3.sum() > B * 0.9
    assert np.all(r["out_accept"][prop3, 1] == 0)
    assert np.all(r["out_tokens"][:, 0] != 3)


def test_race_draw_follows_the_weights_across_chunks():
    V = 4096
    rng = np.random.default_rng(3)
    ids = np.sort(rng.choice(V, size=16, replace=False))
    ids[:4] = [5, 1023, 1024, 4095]       # chunk borders and the ragged tail
    ids = np.unique(ids)
    w = np.zeros(V)
    w[ids] = rng.uniform(0.2, 1.0, size=ids.size)
    draws = []
    for b in range(400):
        for off in range(25):
            x, _, _ = race_draw(w, seed=17, b=b, row=1, offset=off)
            draws.append(x)
    draws = np.array(draws)
    assert set(np.unique(draws)) <= set(ids.tolist())
    assert _chisq_ok(draws, w / w.sum())


def test_race_draw_single_positive_weight_is_deterministic():
    w = np.zeros(3000)
    w[2048 + 7] = 1e-300
    for off in range(20):
        assert race_draw(w, seed=1, b=0, row=0, offset=off)[0] == 2055


def test_explicit_chain_parent_equals_default_chain():
    V, B, N = 50, 64, 5
    x = make_sample_inputs(B, N, V, None, 3.0, draft_noise_std=1.0, seed=51)
    r1 = spec_sample(x["target"], x["draft"], x["tokens"], seed=9, offset=4)
    r2 = spec_sample(x["target"], x["draft"], x["tokens"], parent=chain_parent(N), seed=9, offset=4)
    for key in ("out_tokens", "out_count", "out_path", "out_accept"):
        assert np.array_equal(r1[key], r2[key])


def test_tree_walk_takes_first_accepted_child():
    """Root with children 1,2,3: child 1 can never pass, children 2 and 3 always pass."""
    V, N = 6, 4
    parent = np.array([-1, 0, 0, 0], dtype=np.int32)
    t = torch.zeros(N, V)
    t[0, 0] = -np.inf                     # token 0 has no target mass at the root
    d = t.clone()
    d[0, 0] = 0.0
    d[0, 1:] = 0.0
    B = 300
    tokens = torch.zeros(B, N, dtype=torch.int32)
    tokens[:, 1] = 0                      # rejected for sure
    tokens[:, 2] = 2                      # ratio = Pt/Pd > 1 -> accepted for sure
    tokens[:, 3] = 3
    r = spec_sample(_batch(t, B), _batch(d, B), tokens, parent=parent, seed=4)
    assert np.all(r["out_accept"][:, 1] == 0)
    assert np.all(r["out_accept"][:, 2:] == 1)
    assert np.all(r["out_path"][:, :2] == [0, 2])
    assert np.all(r["out_count"] == 2)
    assert np.all(r["out_tokens"][:, 0] == 2)
    assert np.all(r["stop_row"] == 2) and not np.any(r["residual"])   # node 2 is a leaf: bonus row


def test_tree_outputs_are_consistent_paths():
    N, V, B = 64, 200, 40
    parent = random_tree(N, seed=4321)
    x = make_sample_inputs(B, N, V, parent, 3.0, draft_noise_std=1.0, seed=61)
    r = spec_sample(x["target"], x["draft"], x["tokens"], parent=parent, seed=2, offset=1)
    depth = np.zeros(N, dtype=int)
    for c in range(1, N):
        depth[c] = depth[parent[c]] + 1
    for b in range(B):
        k = r["out_count"][b]
        path = r["out_path"][b, :k]
        assert 1 <= k <= depth.max() + 1
        assert path[0] == 0 and np.all(r["out_path"][b, k:] == -1)
        for a, c in zip(path[:-1], path[1:]):
            assert parent[c] == a and r["out_accept"][b, c] == 1
        assert np.array_equal(r["out_tokens"][b, :k - 1], x["tokens"][b, path[1:]].numpy())
        assert 0 <= r["out_tokens"][b, k - 1] < V and np.all(r["out_tokens"][b, k:] == -1)


def test_offsets_and_seeds_give_independent_rounds():
    V, B, N = 64, 200, 5
    x = make_sample_inputs(B, N, V, None, 3.0, draft_noise_std=1.0, seed=71)
    a = spec_sample(x["target"], x["draft"], x["tokens"], seed=1, offset=0)
    b = spec_sample(x["target"], x["draft"], x["tokens"], seed=1, offset=1)
    c = spec_sample(x["target"], x["draft"], x["tokens"], seed=2, offset=0)
    assert not np.array_equal(a["u"][:, 1:], b["u"][:, 1:])
    assert not np.array_equal(a["u"][:, 1:], c["u"][:, 1:])
    a2 = spec_sample(x["target"], x["draft"], x["tokens"], seed=1, offset=0)
    assert np.array_equal(a["out_tokens"], a2["out_tokens"])


# --- lossless sibling rule -------------------------------------------------------------------

# A tree whose node rows depend only on depth: the root, three children, and two
# children under each of those (N = 10).
_SIB_PARENT = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3])
_SIB_DEPTH = np.array([0, 1, 1, 1, 2, 2, 2, 2, 2, 2])


def test_lossless_chain_equals_first_rule():
    x = make_sample_inputs(300, 5, 700, None, 3.0, draft_noise_std=1.0, seed=41)
    a = spec_sample(x["target"], x["draft"], x["tokens"], seed=7, offset=3)
    b = spec_sample(x["target"], x["draft"], x["tokens"], seed=7, offset=3, siblings="lossless")
    for k in ("out_tokens", "out_count", "out_path"):
        assert np.array_equal(a[k], b[k]), k
    # The lossless walk tests only the nodes it reaches (up to the first rejection).
    for bb in range(300):
        reach = min(int(a["out_count"][bb]) + 1, 5)
        assert np.array_equal(a["out_accept"][bb, :reach], b["out_accept"][bb, :reach])
        assert not b["out_accept"][bb, reach:].any()


def test_lossless_rule_keeps_every_position_on_the_target():
    """Siblings drawn independently from the draft row: each emitted token follows the
    target row of its depth (chi-square), although several siblings compete."""
    V, B = 6, 30000
    t = _rows(V, 3, 1.3, 51)[_SIB_DEPTH]
    d = _rows(V, 3, 1.3, 52)[_SIB_DEPTH]
    x = make_sample_inputs(B, 10, V, _SIB_PARENT, 0, target=_batch(t, B), draft=_batch(d, B),
                           seed=53)
    r = spec_sample(x["target"], x["draft"], x["tokens"], _SIB_PARENT, seed=54, offset=1,
                    siblings="lossless")
    cnt, out = r["out_count"], r["out_tokens"]
    assert np.all((cnt >= 1) & (cnt <= 3))
    for pos in range(3):
        sel = cnt >= pos + 1
        assert _chisq_ok(out[sel, pos], softmax(t[int(np.argmax(_SIB_DEPTH == pos))].double()
                                                 .numpy())), f"position {pos}"


def test_lossless_rule_hand_worked_two_siblings():
    """V = 2, p = (0.9, 0.1), q = (0.5, 0.5), two leaf children both drafting token 1.
    The first test passes with probability 0.2; after its rejection p becomes (1, 0), so
    the second child (token 1) can never pass and the draw is token 0."""
    B = 20000
    t = torch.log(torch.tensor([[0.9, 0.1]] * 3, dtype=torch.float64)).float()
    d = torch.log(torch.tensor([[0.5, 0.5]] * 3, dtype=torch.float64)).float()
    parent = np.array([-1, 0, 0])
    x = make_sample_inputs(B, 3, 2, parent, 0, target=_batch(t, B), draft=_batch(d, B), seed=61)
    x["tokens"][:, 1:] = 1
    r = spec_sample(x["target"], x["draft"], x["tokens"], parent, seed=62, siblings="lossless")
    cnt, path, out = r["out_count"], r["out_path"], r["out_tokens"]
    assert not np.any(path[:, 1] == 2)                 # the second sibling never passes
    assert np.all(out[cnt == 1, 0] == 0)               # after both rejections: token 0
    rate = np.mean(cnt == 2)
    assert abs(rate - 0.2) <= 4 * np.sqrt(0.2 * 0.8 / B)
    # The first-accepted rule tests the second child against p itself: 0.2 + 0.8 * 0.2.
    f = spec_sample(x["target"], x["draft"], x["tokens"], parent, seed=62)
    assert abs(np.mean(f["out_count"] == 2) - 0.36) <= 4 * np.sqrt(0.36 * 0.64 / B)


def test_lossless_first_sibling_test_is_the_plain_ratio():
    parent = random_tree(20, seed=8)
    x = make_sample_inputs(40, 20, 300, parent, 3.0, draft_noise_std=1.0, seed=71)
    a = spec_sample(x["target"], x["draft"], x["tokens"], parent, seed=3)
    b = spec_sample(x["target"], x["draft"], x["tokens"], parent, seed=3, siblings="lossless")
    children = [[c for c in range(20) if parent[c] == u] for u in range(20)]
    for bb in range(40):
        for u in b["out_path"][bb][b["out_path"][bb] >= 0]:
            if children[u]:
                c = children[u][0]
                assert b["ratio"][bb, c] == a["ratio"][bb, c]
