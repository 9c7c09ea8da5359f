"""fp64 attention definitions for the verification step -- test infrastructure.

Plain definitions, no blocking, no online softmax, no splitting:

verify_attention
    "Guide to MagicDec", section 2 "Lossless Target Model Verification Across
    Full Context": the target verifies the drafted tokens with full-context
    attention over all S cached tokens.  "Speculative Decoding in LLM Serving
    Systems", section "The algorithm", step 2: one target pass over
    prefix + drafted tokens yields a distribution at every drafted position,
    so the drafted block is causal within itself.  Same page, section
    "Tree-based variants" (Medusa, SpecInfer) and "Speculative Decoding &
    Medusa Architecture", section 4: a tree of candidates is verified in one
    pass under a mask that lets every token attend only to its ancestors.

    For sequence b, query head h, block node i (0 <= i < n_q):
      hk = h // (Hq/Hkv); L = kv_len[b]; p0 = L - n_q (the block's K/V sit at
      cache positions p0 .. L-1);
      allowed keys = [0, p0)  U  {p0 + t : t an ancestor of i, i included};
      s_j = scale * <q[b,h,i], k[b,hk,j]>, scale = 1/sqrt(D) by default;
      o = sum_j softmax(s)_j v[b,hk,j];   lse = log sum_j exp(s_j).
    A chain is the tree whose node i hangs under i-1.

verify_attention_paged
    The same attention when the cache is a pool of fixed-size pages and a
    block table lists each sequence's pages in order (the serving engines
    "Guide to MagicDec" names for continuous batching, vLLM and
    TensorRT-LLM, keep caches this way): key j of sequence b is row j % P of
    page block_table[b][j // P].  The oracle gathers the pages back into a
    contiguous cache and applies verify_attention.

window_attention
    "Guide to MagicDec", section 1 "Fixed-Window KV Cache Decoupling": the
    draft attends only to the most recent W tokens (a FIFO ring), and "Best
    Practices", item 1: a few dedicated slots keep the first prompt tokens
    (attention sinks).  With T tokens seen (current one included) the keys are
    tokens [0, min(S,T))  U  [max(S, T-W), T).  One query per sequence, so no
    mask inside the window.
"""

from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    """Widen a numpy array or a torch tensor (any float dtype, any device) to float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def ancestors(parent: np.ndarray, i: int) -> list:
    """Node i and all its ancestors under a parent array (parent < 0 marks a root)."""
    out = []
    seen = set()
    while i >= 0:
        if i in seen:
            raise ValueError("parent array has a cycle")
        seen.add(i)
        out.append(i)
        i = int(parent[i])
    return out


def softmax_attention(qrow: np.ndarray, K: np.ndarray, V: np.ndarray,
                      allowed: np.ndarray, scale: float) -> Tuple[np.ndarray, float]:
    """One query row: softmax over the allowed keys of scale*<q,k>, then the weighted sum of V."""
    s = scale * (K @ qrow)
    s = np.where(allowed, s, -np.inf)
    m = np.max(s)
    w = np.exp(s - m)
    tot = np.sum(w)
    return (w @ V) / tot, float(m + np.log(tot))


def verify_attention(q, k, v, kv_len=None, parent=None, scale: Optional[float] = None,
                     heads: Optional[Iterable[Tuple[int, int]]] = None):
    """Block-of-queries attention against the KV cache (chain or tree mask).

    q: [B,Hq,n_q,D]; k, v: [B,Hkv,L_cap,D]; kv_len: [B] (default L_cap);
    parent: None (chain), [n_q] shared by all sequences, or [B,n_q].
    heads: optional iterable of (b, h) to evaluate (others are left NaN).
    Returns (o [B,Hq,n_q,D], lse [B,Hq,n_q]) in float64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, n_q, D = q.shape
    Hkv, L_cap = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None or scale <= 0 else float(scale)
    kv_len = np.full(B, L_cap) if kv_len is None else np.asarray(_f64(kv_len), dtype=np.int64)
    if parent is None:
        par = np.tile(np.arange(-1, n_q - 1), (B, 1))
    else:
        par = np.asarray(_f64(parent), dtype=np.int64)
        if par.ndim == 1:
            par = np.tile(par, (B, 1))
    o = np.full((B, Hq, n_q, D), np.nan)
    lse = np.full((B, Hq, n_q), np.nan)
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    for b, h in todo:
        L = int(kv_len[b])
        if not (n_q <= L <= L_cap):
            raise ValueError("kv_len must lie in [n_q, L_cap]")
        p0 = L - n_q
        hk = h // g
        K = k[b, hk, :L]
        V = v[b, hk, :L]
        for i in range(n_q):
            allowed = np.zeros(L, dtype=bool)
            allowed[:p0] = True
            for t in ancestors(par[b], i):
                allowed[p0 + t] = True
            o[b, h, i], lse[b, h, i] = softmax_attention(q[b, h, i], K, V, allowed, scale)
    return o, lse


def gather_pages(pages, block_table, kv_len, L_max: int):
    """Contiguous [B, Hkv, L_max, D] cache from a page pool [num_pages, Hkv, P, D].

    Key j < kv_len[b] of sequence b is row j % P of page block_table[b][j // P];
    keys at or past kv_len[b] are NaN (verify_attention never reads them).
    """
    bt = np.asarray(_f64(block_table), dtype=np.int64)
    kl = np.asarray(_f64(kv_len), dtype=np.int64)
    _, Hkv, P, D = pages.shape
    B = bt.shape[0]
    out = np.full((B, Hkv, L_max, D), np.nan)
    for b in range(B):
        for j0 in range(0, int(kl[b]), P):           # one page at a time
            n = min(P, int(kl[b]) - j0)
            out[b, :, j0:j0 + n] = _f64(pages[int(bt[b, j0 // P])])[:, :n]
    return out


def verify_attention_paged(q, k_pages, v_pages, block_table, kv_len, L_max: int, parent=None,
                           scale: Optional[float] = None,
                           heads: Optional[Iterable[Tuple[int, int]]] = None):
    """verify_attention over a paged cache (see the module notes)."""
    k = gather_pages(k_pages, block_table, kv_len, L_max)
    v = gather_pages(v_pages, block_table, kv_len, L_max)
    return verify_attention(q, k, v, kv_len, parent=parent, scale=scale, heads=heads)


def window_attention(q, hist_sink_k, hist_sink_v, hist_recent_k, hist_recent_v,
                     total_len, W: int, S: int, scale: Optional[float] = None):
    """One draft-step query per sequence against the sinks and the last W tokens.

    The caches are given chronologically (no ring arithmetic here):
    hist_sink_k/v [B,Hkv,S,D] hold tokens 0..S-1; hist_recent_k/v [B,Hkv,W,D]
    hold tokens T-W .. T-1 in time order (row r is token T-W+r).
    q: [B,Hq,1,D].  Returns (o [B,Hq,1,D], lse [B,Hq,1]) in float64.
    """
    q = _f64(q)
    hr_k = _f64(hist_recent_k)
    hr_v = _f64(hist_recent_v)
    hs_k = _f64(hist_sink_k) if S > 0 else None
    hs_v = _f64(hist_sink_v) if S > 0 else None
    B, Hq, _, D = q.shape
    Hkv = hr_k.shape[1]
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None or scale <= 0 else float(scale)
    T_all = np.asarray(_f64(total_len), dtype=np.int64)
    o = np.zeros((B, Hq, 1, D))
    lse = np.zeros((B, Hq, 1))
    for b in range(B):
        T = int(T_all[b])
        keys_k, keys_v = [], []
        for t in range(0, min(S, T)):              # sink tokens
            keys_k.append(hs_k[b, :, t])
            keys_v.append(hs_v[b, :, t])
        for t in range(max(S, T - W), T):          # window tokens
            r = t - (T - W)
            keys_k.append(hr_k[b, :, r])
            keys_v.append(hr_v[b, :, r])
        Kb = np.stack(keys_k, axis=1)              # [Hkv, n_keys, D]
        Vb = np.stack(keys_v, axis=1)
        allowed = np.ones(Kb.shape[1], dtype=bool)
        for h in range(Hq):
            o[b, h, 0], lse[b, h, 0] = softmax_attention(q[b, h, 0], Kb[h // g], Vb[h // g],
                                                         allowed, scale)
    return o, lse
