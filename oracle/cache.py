"""KV-cache commit after verification -- test infrastructure (oracle side).

"Speculative Decoding in LLM Serving Systems", section "Core idea": guess
ahead, verify, and roll back only what was wrong; "Guide to MagicDec",
step 3 of its reference implementation (the verifier and rollback
controller).  After the acceptance walk, the verified block's cache rows
hold the K/V of every drafted node, accepted or not.  The next round needs
the prefix followed by exactly the accepted path.

Definition (per sequence b, with the block at positions p0 .. p0+n_q-1,
p0 = kv_len[b] - n_q, and the walk's node path[0..count-1], path[0] = 0):
    new_cache[p0 + j] = old_cache[p0 + path[j]]   for j < count,
    new_kv_len[b]     = p0 + count,
everything before p0 unchanged.  For a chain path[j] = j, so only the
length changes.  The draft model's ring got one entry per chain node
0 .. appended-1 this round (the root, then the drafts it fed back); the
entries of nodes that were not accepted are dropped:
    new_total_len[b] = total_len[b] - max(0, appended - count).
A sequence with count 0 (flagged invalid by the sampler) is left as it is.
"""

from __future__ import annotations

import numpy as np


def commit_path(k, v, kv_len, path, count, n_q):
    """Return (k_new, v_new, kv_len_new) as numpy arrays (inputs untouched).

    k, v: [B, Hkv, L_cap, D]; kv_len: [B]; path: [B, N] (-1 padded); count: [B].
    """
    k = np.array(k, copy=True)
    v = np.array(v, copy=True)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    path = np.asarray(path, dtype=np.int64)
    count = np.asarray(count, dtype=np.int64)
    B = k.shape[0]
    new_len = kv_len.copy()
    k_src = k.copy()
    v_src = v.copy()
    for b in range(B):
        c = int(count[b])
        if c < 1:
            continue
        p0 = int(kv_len[b]) - n_q
        rows = [p0 + int(path[b, j]) for j in range(c)]
        k[b, :, p0:p0 + c] = k_src[b][:, rows]
        v[b, :, p0:p0 + c] = v_src[b][:, rows]
        new_len[b] = p0 + c
    return k, v, new_len


def rollback_draft(total_len, count, appended):
    """Draft ring length after dropping the rejected appended drafts."""
    total_len = np.asarray(total_len, dtype=np.int64)
    count = np.asarray(count, dtype=np.int64)
    drop = np.maximum(0, appended - count)
    return np.where(count >= 1, total_len - drop, total_len)
