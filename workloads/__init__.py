"""Seeded synthetic inputs for the speculative verification step.

This module only draws random tensors and lays them out; it holds none of
the verification arithmetic (no attention, no softmax, no acceptance test,
no sampler).  Both the fp64 oracle (under ``oracle/``) and the HIP path
(``long_context_verify_amd``) are fed from here, so the two sides always
see the very same bits.

Shapes follow the workloads the source pages talk about:

* "Guide to MagicDec" (aifetchly blog), section "Fixed-Window KV Cache
  Decoupling" and "Best Practices: Attention Sink Preservation": a target
  cache over the whole context and a draft cache bounded to a window of W
  slots plus a few sink slots.
* "Speculative Decoding & Medusa Architecture" (zyekh blog), section 4
  "Tree-Attention Kernels": a Medusa candidate tree verified in one pass.
* "Speculative Decoding in LLM Serving Systems" (elimelt notes), section
  "The algorithm": a gamma-token chain scored by gamma+1 target rows.

Random draws:

* attention tensors ~ N(0, 1), drawn in fp32 by a seeded torch generator on
  the requested device and rounded once to bf16 (round-to-nearest-even) when
  the workload is bf16;
* target logits ~ N(0, sigma_t) (sigma is a standard deviation), draft
  logits = target + N(0, sigma_n) or independent N(0, sigma_d);
* drafted tokens: node c is drawn from the draft row of its parent with the
  Gumbel-max trick (argmax of logits plus Gumbel noise), which is an exact
  draw from softmax(draft row).  This stands in for the draft model's own
  sampling step, which is not part of the verification step;
* candidate trees: a seeded random parent array with bounded depth and
  branching (numpy PCG64).
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "CONFIGS",
    "make_paged_inputs",
    "WorkloadConfig",
    "chain_parent",
    "random_tree",
    "make_attention_inputs",
    "make_window_inputs",
    "make_sample_inputs",
    "ring_slot_of_token",
]


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    """One synthetic workload (attention layer shape + sampling shape)."""

    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    kv_len: int
    dtype: str            # "f32" or "bf16"
    n_q: int              # query block: gamma+1 for a chain, N nodes for a tree
    tree: bool            # candidate tree (True) or causal chain (False)
    window: Optional[int]  # draft window W (None: no draft window in this config)
    sinks: int
    vocab: int
    target_std: float
    draft_noise_std: Optional[float]   # draft = target + N(0, noise)
    draft_std: Optional[float]         # draft independent N(0, draft_std)
    sample_rows: Optional[int] = None  # sampled nodes per sequence if not n_q
    seed: int = 0

    @property
    def gamma(self) -> int:
        return self.n_q - 1

    @property
    def n_nodes(self) -> int:
        return self.sample_rows if self.sample_rows is not None else self.n_q


# The five workloads.  Names describe the shape; seeds are fixed per workload.
CONFIGS = {
    "tiny_chain": WorkloadConfig(
        name="tiny_chain", batch=1, hq=8, hkv=2, head_dim=64, kv_len=1024,
        dtype="f32", n_q=5, tree=False, window=128, sinks=4, vocab=1000,
        target_std=2.0, draft_noise_std=None, draft_std=2.0, seed=1001),
    "llama8b_32k_chain": WorkloadConfig(
        name="llama8b_32k_chain", batch=8, hq=32, hkv=8, head_dim=128,
        kv_len=32768, dtype="bf16", n_q=5, tree=False, window=512, sinks=4,
        vocab=128256, target_std=3.0, draft_noise_std=1.0, draft_std=None,
        seed=1002),
    "magicdec_128k_chain": WorkloadConfig(
        name="magicdec_128k_chain", batch=4, hq=32, hkv=8, head_dim=128,
        kv_len=131072, dtype="bf16", n_q=6, tree=False, window=256, sinks=4,
        vocab=128256, target_std=3.0, draft_noise_std=1.5, draft_std=None,
        seed=1003),
    "medusa_tree64_8k": WorkloadConfig(
        name="medusa_tree64_8k", batch=16, hq=32, hkv=8, head_dim=128,
        kv_len=8192, dtype="bf16", n_q=64, tree=True, window=None, sinks=4,
        vocab=32000, target_std=3.0, draft_noise_std=1.0, draft_std=None,
        seed=1004),
    "llama70b_16k_chain_b64": WorkloadConfig(
        name="llama70b_16k_chain_b64", batch=64, hq=64, hkv=8, head_dim=128,
        kv_len=16384, dtype="bf16", n_q=4, tree=False, window=None, sinks=4,
        vocab=128256, target_std=3.0, draft_noise_std=1.0, draft_std=None,
        seed=1005),
}

TREE_SEED = 4321


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, std, gen, device, dtype):
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def chain_parent(n: int) -> np.ndarray:
    """Parent array of a chain of n nodes: node c hangs under c-1, node 0 is the root."""
    p = np.arange(-1, n - 1, dtype=np.int32)
    return p


def random_tree(n: int, max_depth: int = 5, max_children: int = 4,
                seed: int = TREE_SEED) -> np.ndarray:
    """Seeded random candidate tree as a parent array (parent[c] < c, parent[0] = -1).

    Node 0 is the root at depth 0.  Each later node picks its parent uniformly
    among earlier nodes whose depth is below ``max_depth`` and that have fewer
    than ``max_children`` children (numpy PCG64).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    parent = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int64)
    nchild = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        cand = [j for j in range(i) if depth[j] < max_depth and nchild[j] < max_children]
        if not cand:
            raise ValueError("tree limits leave no free parent")
        j = cand[int(rng.integers(len(cand)))]
        parent[i] = j
        depth[i] = depth[j] + 1
        nchild[j] += 1
    return parent


def make_attention_inputs(B: int, Hq: int, Hkv: int, n_q: int, D: int, L: int,
                          dtype: str = "bf16", seed: int = 0, device="cpu",
                          L_cap: Optional[int] = None,
                          kv_len: Optional[Sequence[int]] = None):
    """Q [B,Hq,n_q,D] and K/V caches [B,Hkv,L_cap,D] ~ N(0,1), plus kv_len [B] int32.

    ``kv_len[b]`` counts the n_q block tokens, whose K/V already sit at cache
    positions kv_len-n_q .. kv_len-1.  Slots at or past kv_len hold random
    values too (they must never influence the result).
    """
    L_cap = L if L_cap is None else L_cap
    if kv_len is None:
        kv_len = [L] * B
    g = _gen(device, seed)
    q = _normal((B, Hq, n_q, D), 1.0, g, device, dtype)
    k = _normal((B, Hkv, L_cap, D), 1.0, g, device, dtype)
    v = _normal((B, Hkv, L_cap, D), 1.0, g, device, dtype)
    kl = torch.tensor(list(kv_len), dtype=torch.int32, device=device)
    return {"q": q, "k": k, "v": v, "kv_len": kl, "L_cap": L_cap}


def make_paged_inputs(k, v, kv_len, page_size: int, seed: int = 0, spare_pages: int = 3,
                      junk: float = 50.0):
    """Scatter contiguous caches [B, Hkv, L_cap, D] into a shuffled page pool.

    Returns dict(k_pages, v_pages [num_pages, Hkv, P, D], block_table [B, stride]
    int32, stride = ceil(L_cap / P)).  Sequence b gets ceil(kv_len[b] / P) pages
    at seeded random pool positions (numpy PCG64); table entries past those are
    -1 and the spare pages hold ``junk``, so a read outside the table shows.
    """
    B, Hkv, L_cap, D = k.shape
    P = int(page_size)
    kl = [int(x) for x in (kv_len.tolist() if hasattr(kv_len, "tolist") else kv_len)]
    need = [(L + P - 1) // P for L in kl]
    num_pages = sum(need) + spare_pages
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(num_pages)
    stride = (L_cap + P - 1) // P
    table = np.full((B, stride), -1, dtype=np.int32)
    kp = torch.full((num_pages, Hkv, P, D), junk, dtype=k.dtype, device=k.device)
    vp = torch.full((num_pages, Hkv, P, D), -junk, dtype=v.dtype, device=v.device)
    nxt = 0
    for b in range(B):
        for i in range(need[b]):
            pid = int(perm[nxt])
            nxt += 1
            table[b, i] = pid
            lo, hi = i * P, min((i + 1) * P, L_cap)
            kp[pid, :, :hi - lo] = k[b, :, lo:hi]
            vp[pid, :, :hi - lo] = v[b, :, lo:hi]
    bt = torch.as_tensor(table, device=k.device)
    return {"k_pages": kp, "v_pages": vp, "block_table": bt, "stride": stride}


def ring_slot_of_token(t: int, W: int, S: int) -> int:
    """Physical ring slot of token t >= S in a W-slot FIFO ring behind S sink slots."""
    if t < S:
        raise ValueError("sink tokens do not live in the ring")
    return (t - S) % W


def make_window_inputs(B: int, Hq: int, Hkv: int, D: int, W: int, S: int,
                       total_len: Sequence[int], dtype: str = "bf16",
                       seed: int = 0, device="cpu", fused_append: bool = False):
    """Draft-cache inputs for one draft step with a W-slot ring and S sink slots.

    For each sequence b with T = total_len[b] tokens seen so far (the current
    token included), the retained tokens are the first min(S, T) tokens (sink
    slots) and the last min(W, T-S) tokens (ring slots).  Returned are both
    the physical buffers (ring written through the FIFO slot map
    ``ring_slot_of_token``) and the chronological copy of the retained tokens:

    * ``hist_sink_k/v``  [B,Hkv,S,D]   tokens 0..S-1 (rows >= T unused)
    * ``hist_recent_k/v`` [B,Hkv,W,D]  tokens T-W .. T-1 in time order
      (row r holds token T-W+r; rows whose token is < S are unused)

    With ``fused_append`` the current token T-1 is handed separately as
    k_new/v_new [B,Hkv,1,D] and its physical slot holds stale random data.
    """
    g = _gen(device, seed)
    q = _normal((B, Hq, 1, D), 1.0, g, device, dtype)
    hs_k = _normal((B, Hkv, S, D), 1.0, g, device, dtype) if S > 0 else None
    hs_v = _normal((B, Hkv, S, D), 1.0, g, device, dtype) if S > 0 else None
    hr_k = _normal((B, Hkv, W, D), 1.0, g, device, dtype)
    hr_v = _normal((B, Hkv, W, D), 1.0, g, device, dtype)
    stale_k = _normal((B, Hkv, W, D), 1.0, g, device, dtype)
    stale_v = _normal((B, Hkv, W, D), 1.0, g, device, dtype)
    stale_sk = _normal((B, Hkv, max(S, 1), D), 1.0, g, device, dtype)
    stale_sv = _normal((B, Hkv, max(S, 1), D), 1.0, g, device, dtype)

    k_ring = stale_k.clone()
    v_ring = stale_v.clone()
    k_sink = stale_sk[:, :, :S].clone() if S > 0 else None
    v_sink = stale_sv[:, :, :S].clone() if S > 0 else None
    k_new = v_new = None
    if fused_append:
        k_new = torch.empty((B, Hkv, 1, D), dtype=q.dtype, device=device)
        v_new = torch.empty((B, Hkv, 1, D), dtype=q.dtype, device=device)
    for b, T in enumerate(total_len):
        T = int(T)
        if T < 1:
            raise ValueError("total_len must be >= 1")
        last = T - 1 if fused_append else T
        # sink tokens 0 .. min(S,T)-1 (the current token is handed over separately)
        ns = min(S, last)
        if ns > 0:
            k_sink[b, :, :ns] = hs_k[b, :, :ns]
            v_sink[b, :, :ns] = hs_v[b, :, :ns]
        # ring tokens max(S, T-W) .. T-1; chronological row r <-> token T-W+r
        toks = list(range(max(S, T - W), last))
        if toks:
            rows = torch.tensor([t - (T - W) for t in toks], device=device)
            slots = torch.tensor([ring_slot_of_token(t, W, S) for t in toks], device=device)
            k_ring[b, :, slots] = hr_k[b, :, rows]
            v_ring[b, :, slots] = hr_v[b, :, rows]
        if fused_append:
            if T - 1 < S:
                k_new[b, :, 0] = hs_k[b, :, T - 1]
                v_new[b, :, 0] = hs_v[b, :, T - 1]
            else:
                k_new[b, :, 0] = hr_k[b, :, W - 1]
                v_new[b, :, 0] = hr_v[b, :, W - 1]
    tl = torch.tensor([int(t) for t in total_len], dtype=torch.int32, device=device)
    return {
        "q": q, "k_ring": k_ring, "v_ring": v_ring, "k_sink": k_sink,
        "v_sink": v_sink, "k_new": k_new, "v_new": v_new, "total_len": tl,
        "hist_sink_k": hs_k, "hist_sink_v": hs_v,
        "hist_recent_k": hr_k, "hist_recent_v": hr_v,
        "W": W, "S": S,
    }


def make_sample_inputs(B: int, N: int, V: int, parent: Optional[np.ndarray],
                       target_std: float, draft_noise_std: Optional[float] = None,
                       draft_std: Optional[float] = None, seed: int = 0,
                       device="cpu", target=None, draft=None):
    """Target/draft logits [B,N,V] fp32 and drafted tokens [B,N] int32.

    Row u of ``target`` holds the target model's next-token logits at node u;
    row u of ``draft`` the draft logits from which u's children were drawn.
    Token c (c >= 1) is drawn from softmax(draft[b, parent[c]]) by Gumbel-max;
    tokens[:, 0] is the last accepted token and is set to 0 (unused).
    ``target``/``draft`` may be supplied to reuse fixed logits.
    """
    g = _gen(device, seed)
    if parent is None:
        parent = chain_parent(N)
    parent = np.asarray(parent, dtype=np.int64)
    if target is None:
        target = torch.randn(B, N, V, generator=g, device=device) * target_std
    if draft is None:
        if draft_noise_std is not None:
            draft = target + torch.randn(B, N, V, generator=g, device=device) * draft_noise_std
        else:
            draft = torch.randn(B, N, V, generator=g, device=device) * draft_std
    target = target.to(torch.float32).contiguous()
    draft = draft.to(torch.float32).contiguous()
    tokens = torch.zeros(B, N, dtype=torch.int32, device=device)
    if N > 1:
        par = torch.as_tensor(parent[1:], device=device)
        rows = draft[:, par, :]                       # [B, N-1, V]
        u = torch.rand(rows.shape, generator=g, device=device, dtype=torch.float64)
        u = u.clamp_(min=1e-300)
        gumbel = -torch.log(-torch.log(u))
        tokens[:, 1:] = torch.argmax(rows.to(torch.float64) + gumbel, dim=-1).to(torch.int32)
    return {"target": target, "draft": draft, "tokens": tokens,
            "parent": np.asarray(parent, dtype=np.int32)}
