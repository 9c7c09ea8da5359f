"""Pins of the oracle's verify and window attention (CPU only).

Each test ties the oracle to something other than itself: torch's float64
scaled_dot_product_attention (a library routine), closed forms (constant
keys), brute-force reductions (tree row = chain over the root-to-node path),
or an independent FIFO simulation for the draft window.
"""

import collections

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.attention import (ancestors, gather_pages, verify_attention, verify_attention_paged,
                              window_attention)
from workloads import (chain_parent, make_attention_inputs, make_paged_inputs, make_window_inputs,
                       random_tree)


def _sdpa_last_rows(q_rows, K, V, n_q):
    """Last n_q rows of full causal self-attention over L tokens, via torch float64 SDPA.

    q_rows [Hq, n_q, D] are the queries of the last n_q tokens; K, V [Hq, L, D].
    A square L x L causal call is made (is_causal is top-left aligned), with
    zero queries for the first L-n_q tokens; only the last n_q rows are kept.
    """
    Hq, L, D = K.shape
    Q = torch.zeros(Hq, L, D, dtype=torch.float64)
    Q[:, L - n_q:] = q_rows
    out = F.scaled_dot_product_attention(Q[None], K[None], V[None], is_causal=True)[0]
    return out[:, L - n_q:]


@pytest.mark.parametrize("B,Hq,Hkv,n_q,D,L", [(2, 8, 2, 5, 64, 300), (1, 4, 4, 1, 32, 17),
                                             (1, 6, 3, 6, 16, 6)])
def test_chain_equals_causal_sdpa_with_gqa(B, Hq, Hkv, n_q, D, L):
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, L, dtype="f32", seed=5)
    o, lse = verify_attention(x["q"], x["k"], x["v"], x["kv_len"])
    g = Hq // Hkv
    for b in range(B):
        K = x["k"][b].double().repeat_interleave(g, dim=0)     # GQA -> MHA
        V = x["v"][b].double().repeat_interleave(g, dim=0)
        ref = _sdpa_last_rows(x["q"][b].double(), K, V, n_q)
        np.testing.assert_allclose(o[b], ref.numpy(), rtol=0, atol=1e-12)


def test_ragged_kv_len_and_unused_slots():
    x = make_attention_inputs(3, 4, 2, 4, 32, 64, dtype="f32", seed=9, L_cap=80,
                              kv_len=[64, 4, 80])
    o, _ = verify_attention(x["q"], x["k"], x["v"], x["kv_len"])
    for b, L in enumerate([64, 4, 80]):
        K = x["k"][b, :, :L].double().repeat_interleave(2, dim=0)
        V = x["v"][b, :, :L].double().repeat_interleave(2, dim=0)
        ref = _sdpa_last_rows(x["q"][b].double(), K, V, 4)
        np.testing.assert_allclose(o[b], ref.numpy(), rtol=0, atol=1e-12)


def test_chain_parent_array_equals_default_chain():
    x = make_attention_inputs(1, 4, 2, 6, 16, 40, dtype="f32", seed=3)
    o1, l1 = verify_attention(x["q"], x["k"], x["v"])
    o2, l2 = verify_attention(x["q"], x["k"], x["v"], parent=chain_parent(6))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_lse_closed_form_with_constant_keys():
    """All keys equal -> every allowed score is the same s, so lse = s + ln(#allowed)."""
    B, Hq, Hkv, n_q, D, L = 1, 2, 1, 5, 8, 50
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, L, dtype="f32", seed=4)
    k = torch.zeros_like(x["k"])
    k[..., :] = x["k"][0, 0, 0]
    _, lse = verify_attention(x["q"], k, x["v"])
    for h in range(Hq):
        for i in range(n_q):
            s = float(x["q"][0, h, i].double() @ k[0, 0, 0].double()) / np.sqrt(D)
            assert abs(lse[0, h, i] - (s + np.log(L - n_q + i + 1))) < 1e-12


def test_tree_row_equals_chain_over_its_path():
    """Tree node i sees the prefix plus its root-to-i path: the same as a chain over that path."""
    n, D, L0 = 24, 16, 37
    parent = random_tree(n, max_depth=4, max_children=3, seed=17)
    x = make_attention_inputs(1, 4, 2, n, D, L0 + n, dtype="f32", seed=21)
    o, lse = verify_attention(x["q"], x["k"], x["v"], parent=parent)
    for i in range(n):
        path = ancestors(parent, i)[::-1]                 # root .. i
        idx = list(range(L0)) + [L0 + t for t in path]
        K = x["k"][:, :, idx]
        V = x["v"][:, :, idx]
        qi = x["q"][:, :, i:i + 1]
        oc, lc = verify_attention(qi, K, V)               # a single query at the end
        np.testing.assert_allclose(o[0, :, i], oc[0, :, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, :, i], lc[0, :, 0], rtol=0, atol=1e-12)
        # and that chain itself is plain softmax attention (library routine)
        ref = F.scaled_dot_product_attention(qi[0].double()[None], K[0].double().repeat_interleave(2, 0)[None],
                                             V[0].double().repeat_interleave(2, 0)[None])[0]
        np.testing.assert_allclose(o[0, :, i], ref[:, 0].numpy(), rtol=0, atol=1e-12)


def test_forest_of_roots_sees_prefix_and_itself():
    n, D, L0 = 7, 8, 20
    parent = np.full(n, -1, dtype=np.int32)
    x = make_attention_inputs(1, 2, 1, n, D, L0 + n, dtype="f32", seed=8)
    o, _ = verify_attention(x["q"], x["k"], x["v"], parent=parent)
    for i in range(n):
        idx = list(range(L0)) + [L0 + i]
        ref = F.scaled_dot_product_attention(x["q"][:, :, i:i + 1].double(),
                                             x["k"][:, :, idx].double().expand(1, 2, -1, -1),
                                             x["v"][:, :, idx].double().expand(1, 2, -1, -1))
        np.testing.assert_allclose(o[0, :, i], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_constant_key_probe_counts_allowed_keys():
    """Equal keys -> output = mean of the allowed V rows; V = one-hot position reveals the set."""
    n, L0 = 16, 10
    parent = random_tree(n, max_depth=3, max_children=4, seed=99)
    L = L0 + n
    D = L                                    # one channel per cache position
    q = torch.randn(1, 1, n, D, dtype=torch.float64)
    k = torch.ones(1, 1, L, D, dtype=torch.float64)
    v = torch.eye(L, dtype=torch.float64)[None, None]
    o, _ = verify_attention(q, k, v, parent=parent)
    for i in range(n):
        allowed = set(range(L0)) | {L0 + t for t in ancestors(parent, i)}
        expect = np.array([1.0 / len(allowed) if j in allowed else 0.0 for j in range(L)])
        np.testing.assert_allclose(o[0, 0, i], expect, rtol=0, atol=1e-14)


def test_mask_leak_probe_tree():
    """Channel 0 of V is 1 only on block keys a query must not see -> that query outputs exactly 0."""
    n, D, L0 = 12, 4, 9
    parent = random_tree(n, max_depth=3, max_children=2, seed=5)
    x = make_attention_inputs(1, 2, 1, n, D, L0 + n, dtype="f32", seed=6)
    for i in range(n):
        anc = set(ancestors(parent, i))
        v = x["v"].clone()
        v[..., 0] = 0.0
        for t in range(n):
            if t not in anc:
                v[0, 0, L0 + t, 0] = 1.0
        o, _ = verify_attention(x["q"], x["k"], v, parent=parent)
        assert np.all(o[0, :, i, 0] == 0.0)


def _fifo_keys(T, W, S):
    """Independent model of the draft cache: S sink slots, then a bounded deque of W slots."""
    sinks, ring = [], collections.deque(maxlen=W)
    for t in range(T):
        if len(sinks) < S:
            sinks.append(t)
        else:
            ring.append(t)
    return sinks + list(ring)


@pytest.mark.parametrize("T", [1, 3, 4, 5, 20, 36, 37, 100, 131])
def test_window_equals_sdpa_over_fifo_tokens(T):
    B, Hq, Hkv, D, W, S = 1, 4, 2, 16, 32, 4
    x = make_window_inputs(B, Hq, Hkv, D, W, S, [T], dtype="f32", seed=T)
    o, lse = window_attention(x["q"], x["hist_sink_k"], x["hist_sink_v"], x["hist_recent_k"],
                              x["hist_recent_v"], x["total_len"], W, S)
    toks = _fifo_keys(T, W, S)

    def tok_kv(t):
        if t < S:
            return x["hist_sink_k"][0, :, t], x["hist_sink_v"][0, :, t]
        return x["hist_recent_k"][0, :, t - (T - W)], x["hist_recent_v"][0, :, t - (T - W)]

    K = torch.stack([tok_kv(t)[0] for t in toks], dim=1).double().repeat_interleave(2, 0)
    V = torch.stack([tok_kv(t)[1] for t in toks], dim=1).double().repeat_interleave(2, 0)
    ref = F.scaled_dot_product_attention(x["q"][0].double()[None], K[None], V[None])[0]
    np.testing.assert_allclose(o[0, :, 0], ref[:, 0].numpy(), rtol=0, atol=1e-12)
    if T <= S + W:
        assert len(toks) == T           # the window covers the whole history: full attention


def test_window_ring_buffer_holds_the_fifo_tokens():
    """The physical ring written by the generator decodes back to the FIFO's retained tokens."""
    W, S = 8, 2
    for T in range(1, 40):
        x = make_window_inputs(1, 1, 1, 4, W, S, [T], dtype="f32", seed=T)
        toks = _fifo_keys(T, W, S)
        ring_toks = [t for t in toks if t >= S]
        # each retained ring token sits in a distinct slot, and that slot holds its K row
        slots = [(t - S) % W for t in ring_toks]
        assert len(set(slots)) == len(slots)
        for t, s in zip(ring_toks, slots):
            assert torch.equal(x["k_ring"][0, 0, s], x["hist_recent_k"][0, 0, t - (T - W)])
        for t in toks:
            if t < S:
                assert torch.equal(x["k_sink"][0, 0, t], x["hist_sink_k"][0, 0, t])


def test_window_is_flat_in_context_length():
    """Only S + W keys are ever touched: huge T with the same retained tokens gives the same output."""
    W, S = 16, 4
    a = make_window_inputs(1, 2, 1, 8, W, S, [1000], dtype="f32", seed=1)
    o1, _ = window_attention(a["q"], a["hist_sink_k"], a["hist_sink_v"], a["hist_recent_k"],
                             a["hist_recent_v"], [1000], W, S)
    o2, _ = window_attention(a["q"], a["hist_sink_k"], a["hist_sink_v"], a["hist_recent_k"],
                             a["hist_recent_v"], [10**6], W, S)
    assert np.array_equal(o1, o2)


def test_gather_pages_hand_worked():
    """P = 3: sequence 0 lives on pages 2 then 0, sequence 1 on page 1."""
    pages = np.zeros((3, 1, 3, 1))
    pages[2, 0, :, 0] = [10, 11, 12]
    pages[0, 0, :, 0] = [13, 14, 15]
    pages[1, 0, :, 0] = [20, 21, 22]
    bt = np.array([[2, 0], [1, -1]])
    out = gather_pages(pages, bt, [5, 2], L_max=6)
    assert out[0, 0, :5, 0].tolist() == [10, 11, 12, 13, 14]
    assert out[1, 0, :2, 0].tolist() == [20, 21]
    assert np.isnan(out[0, 0, 5, 0]) and np.isnan(out[1, 0, 2:, 0]).all()


@pytest.mark.parametrize("P,tree", [(64, False), (4, True), (7, False)])
def test_paged_equals_contiguous(P, tree):
    """A shuffled page pool with a block table gives the contiguous result."""
    B, Hq, Hkv, n_q, D, L = 3, 4, 2, 6, 16, 150
    kv = [150, 97, 6]
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, L, dtype="f32", seed=8, kv_len=kv)
    parent = random_tree(n_q, seed=3) if tree else None
    pg = make_paged_inputs(x["k"], x["v"], x["kv_len"], P, seed=1)
    o1, l1 = verify_attention(x["q"], x["k"], x["v"], x["kv_len"], parent=parent)
    o2, l2 = verify_attention_paged(x["q"], pg["k_pages"], pg["v_pages"], pg["block_table"],
                                    x["kv_len"], L, parent=parent)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # Entries past each sequence's pages are -1 and never needed.
    bt = pg["block_table"].numpy()
    for b in range(B):
        need = (kv[b] + P - 1) // P
        assert (bt[b, :need] >= 0).all() and (bt[b, need:] == -1).all()


@pytest.mark.parametrize("T", [1, 3, 4, 5, 20, 36, 37, 100])
def test_window_constant_keys_count_the_attended_tokens(T):
    """Equal keys: lse - score = ln(min(S, T) + min(W, T - S))."""
    W, S, D = 32, 4, 8
    x = make_window_inputs(1, 2, 1, D, W, S, [T], dtype="f32", seed=T)
    kconst = torch.full((D,), 0.25)
    for name in ("hist_sink_k", "hist_recent_k"):
        x[name][:] = kconst
    _, lse = window_attention(x["q"], x["hist_sink_k"], x["hist_sink_v"], x["hist_recent_k"],
                              x["hist_recent_v"], x["total_len"], W, S)
    s = (x["q"][0, :, 0].double() @ kconst.double()).numpy() / np.sqrt(D)
    count = min(S, T) + min(W, max(T - S, 0))
    np.testing.assert_allclose(lse[0, :, 0] - s, np.log(count), rtol=0, atol=1e-12)
