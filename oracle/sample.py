"""fp64 speculative-sampling tail (accept / resample / bonus) -- test infrastructure.

What is computed, and where the pages state it:

* softmax of the target and draft logits over the vocabulary
  ("Speculative Decoding & Medusa Architecture", section 2 code; "Guide to
  MagicDec", verifier step 3);
* drafted token x at node c is accepted with probability
  min(1, p_target(x) / p_draft(x)), both taken at c's parent ("Guide to
  MagicDec", section 2, acceptance equation; "Speculative Decoding in LLM
  Serving Systems", section "Accepting and rejecting": accept outright when
  the target likes x at least as much as the draft, else with the ratio);
* drafted tokens are walked from the root; at the first rejection the rest is
  discarded and one token is drawn from the normalised max(p_target -
  p_draft, 0) at that position ("Guide to MagicDec", resampling equation;
  same notes, "Accepting and rejecting");
* if every drafted token on the walk is accepted, one bonus token is drawn
  from the target distribution after the last one (same notes: between 1 and
  gamma+1 tokens per round; "Guide to MagicDec", verifier step 3).

Readings taken where the pages leave a step open (each listed in the design
notes of the repository):

* node view: node 0 is the last accepted token, nodes 1..N-1 are drafted
  tokens with parent[c] < c; a chain is parent[c] = c-1.  Target row u holds
  the target distribution after node u, draft row u the draft distribution
  from which u's children were drawn;
* every node c >= 1 gets its own uniform u_c = U(philox(c, 0, b, 4*offset));
  acc_c = u_c < ratio_c (strict: u in (0,1), so ratio >= 1 always accepts and
  a token the target gives zero mass never does); no clamps on p_draft;
* the walk takes, at each node, the first child (lowest index) that passed its
  test; for a chain this is exactly "stop at the first rejection";
* residual weights max(Pt - Pd, 0); if they sum to zero, Pt is used;
* with ``siblings="lossless"`` (a rule the pages name through SpecInfer's
  tree verification but do not spell out) the children of a node are tested
  in index order against a distribution that is updated after each
  rejection: p_0 = the target row, and after child i is rejected
  p_i = normalised max(p_{i-1} - q, 0), q the draft row of the node.  The
  first child with u_c < p_{i-1}(x_c) / q(x_c) is taken; if all are
  rejected the draw comes from the last p_i.  When the children's tokens were
  drawn independently from q this keeps every emitted token distributed as
  the target (multi-round speculative sampling); for a chain it is the rule
  above;
* the draw from a weight vector w is a two-level exponential race: chunks of
  1024 ids compete with score W_c / E1_c, E1_c = -ln U(philox(c, row, b,
  4*offset+2), word 0); inside the winning chunk ids compete with score
  w_x / E2_x, E2_x = -ln U(philox(x // 4, row, b, 4*offset+3), word x % 4);
  ties go to the lowest index.  Exponential races pick index i with
  probability w_i / sum(w), so the draw is exact in distribution.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .philox import philox4x32, seed_key, uniform24

RACE_CHUNK = 1024
STREAM_ACCEPT = 0
STREAM_RACE_CHUNK = 2
STREAM_RACE_ID = 3

TIE_BAND = 1e-6          # |ratio - u| at or below this is a floating-point near-tie
RACE_MARGIN = 1e-5       # best/second race score at or below 1 + this is a near-tie
WSUM_FLOOR = 1e-6        # residual mass at or below this sits at the fallback boundary


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def softmax(x: np.ndarray) -> np.ndarray:
    """Max-shifted softmax of one row in float64 (-inf entries get probability 0)."""
    m = np.max(x)
    e = np.exp(x - m)
    return e / np.sum(e)


def uniforms(seed: int, c0, c1, c2, c3, word=0) -> np.ndarray:
    """Uniforms in (0,1) from Philox4x32-10 at counter (c0,c1,c2,c3), output word ``word``."""
    k0, k1 = seed_key(seed)
    out = philox4x32(c0, c1, c2, c3, k0, k1)
    words = np.stack(np.broadcast_arrays(*out), axis=0)
    word = np.broadcast_to(np.asarray(word, dtype=np.int64), words.shape[1:])
    picked = np.take_along_axis(words, word[None, ...], axis=0)[0]
    return uniform24(picked)


def _top2_ratio(scores: np.ndarray) -> float:
    fin = scores[np.isfinite(scores) & (scores > 0)]
    if fin.size < 2:
        return np.inf
    top = np.sort(fin)[-2:]
    return float(top[1] / top[0])


def race_draw(w: np.ndarray, seed: int, b: int, row: int, offset: int,
              chunk: int = RACE_CHUNK):
    """Two-level exponential race over weights w >= 0 (not necessarily normalised).

    Returns (index, level-1 top-2 score ratio, level-2 top-2 score ratio).
    """
    V = w.shape[0]
    nch = (V + chunk - 1) // chunk
    Wc = np.array([np.sum(w[c * chunk:(c + 1) * chunk]) for c in range(nch)])
    cidx = np.arange(nch)
    E1 = -np.log(uniforms(seed, cidx, row, b, 4 * offset + STREAM_RACE_CHUNK, 0))
    s1 = np.where(Wc > 0, Wc / E1, -np.inf)
    cstar = int(np.argmax(s1))           # first maximum = lowest index on ties
    xs = np.arange(cstar * chunk, min(V, (cstar + 1) * chunk))
    E2 = -np.log(uniforms(seed, xs // 4, row, b, 4 * offset + STREAM_RACE_ID, xs % 4))
    wx = w[xs]
    s2 = np.where(wx > 0, wx / E2, -np.inf)
    x = int(xs[int(np.argmax(s2))])
    return x, _top2_ratio(s1), _top2_ratio(s2)


def spec_sample(target_logits, draft_logits, tokens, parent=None, seed: int = 0,
                offset: int = 0, chunk: int = RACE_CHUNK, siblings: str = "first"):
    """Accept/resample/bonus for a batch of chains or candidate trees.

    target_logits, draft_logits: [B,N,V]; tokens: [B,N] (tokens[:,0] unused);
    parent: None (chain), [N] shared, or [B,N] (parent[0] = -1, parent[c] < c).
    Returns a dict of numpy arrays:
      out_tokens [B,N] int32 (accepted drafted tokens, then the drawn token,
      -1 padded), out_count [B] int32, out_path [B,N] int32 (-1 padded),
      out_accept [B,N] uint8 (per-node test; node 0 reported as 1),
    and per-sequence diagnostics: ratio [B,N], u [B,N], stop_row [B],
    residual [B] bool, wsum [B], margin1 [B], margin2 [B], exempt [B] bool.
    siblings: "first" (each node tested against the target row; the walk takes
    the first child that passed) or "lossless" (see the module notes).
    """
    if siblings not in ("first", "lossless"):
        raise ValueError("siblings must be 'first' or 'lossless'")
    t = _f64(target_logits)
    d = _f64(draft_logits)
    tok = np.asarray(_f64(tokens), dtype=np.int64)
    B, N, V = t.shape
    if parent is None:
        par_all = np.tile(np.arange(-1, N - 1), (B, 1))
    else:
        par_all = np.asarray(_f64(parent), dtype=np.int64)
        if par_all.ndim == 1:
            par_all = np.tile(par_all, (B, 1))

    out_tokens = np.full((B, N), -1, dtype=np.int32)
    out_path = np.full((B, N), -1, dtype=np.int32)
    out_count = np.zeros(B, dtype=np.int32)
    out_accept = np.zeros((B, N), dtype=np.uint8)
    ratio_all = np.full((B, N), np.nan)
    u_all = np.full((B, N), np.nan)
    stop_row = np.zeros(B, dtype=np.int64)
    residual = np.zeros(B, dtype=bool)
    wsum = np.full(B, np.nan)
    margin1 = np.full(B, np.inf)
    margin2 = np.full(B, np.inf)
    exempt = np.zeros(B, dtype=bool)

    for b in range(B):
        par = par_all[b]
        if par[0] >= 0 or np.any(par[1:] >= np.arange(1, N)) or np.any(par[1:] < 0):
            raise ValueError("parent array must be a single-rooted tree with parent[c] < c")
        children = [[] for _ in range(N)]
        for c in range(1, N):
            children[int(par[c])].append(c)
        Pt = {}
        Pd = {}
        for u in range(N):
            if children[u]:
                Pt[u] = softmax(t[b, u])
                Pd[u] = softmax(d[b, u])

        # per-node uniforms from the counter-based generator
        cs = np.arange(1, N)
        uc = uniforms(seed, cs, 0, b, 4 * offset + STREAM_ACCEPT, 0) if N > 1 else np.zeros(0)
        for c in range(1, N):
            if not (0 <= int(tok[b, c]) < V):
                raise ValueError("drafted token out of range")
            u_all[b, c] = uc[c - 1]

        def ratio_of(pnum, pden):
            if pden > 0:
                return pnum / pden
            return np.inf if pnum > 0 else 0.0

        near_tie = False
        small_mass = False
        acc = np.zeros(N, dtype=bool)
        acc[0] = True
        if siblings == "first":
            # every node tested against its parent's rows; the walk takes the
            # first child (index order) that passed
            for c in range(1, N):
                p = int(par[c])
                x = int(tok[b, c])
                ratio_all[b, c] = ratio_of(Pt[p][x], Pd[p][x])
                acc[c] = uc[c - 1] < ratio_all[b, c]
            cur = 0
            path = [0]
            while True:
                nxt = None
                for c in children[cur]:
                    if abs(ratio_all[b, c] - u_all[b, c]) <= TIE_BAND:
                        near_tie = True
                    if acc[c]:
                        nxt = c
                        break
                if nxt is None:
                    break
                path.append(nxt)
                cur = nxt
            # stop row: residual after a rejection, target distribution at a leaf
            if children[cur]:
                w = np.maximum(Pt[cur] - Pd[cur], 0.0)
                residual[b] = True
                wsum[b] = float(np.sum(w))
                if wsum[b] <= 0.0:
                    w = Pt[cur]
            else:
                w = softmax(t[b, cur])
                wsum[b] = 1.0
        else:
            # siblings tested in index order against p_i, updated after each rejection
            cur = 0
            path = [0]
            while True:
                if not children[cur]:
                    w = softmax(t[b, cur])
                    wsum[b] = 1.0
                    break
                q = Pd[cur]
                p_i = Pt[cur]
                # p_i = max(p - shift q, 0) / mass in closed form; only used to size
                # the near-tie band (a kernel evaluating that form in fp32 sums
                # carries an error of about 1e-7 (p(x)/q(x) + 2 shift) / mass)
                shift, mass = 0.0, 1.0
                nxt = None
                for c in children[cur]:
                    x = int(tok[b, c])
                    r = ratio_of(p_i[x], q[x])
                    ratio_all[b, c] = r
                    scale = 1.0
                    if q[x] > 0 and np.isfinite(r):
                        scale = max(1.0, (Pt[cur][x] / q[x] + 2.0 * shift) / mass + r)
                    if abs(r - uc[c - 1]) <= TIE_BAND * scale:
                        near_tie = True
                    if uc[c - 1] < r:
                        acc[c] = True
                        nxt = c
                        break
                    res = np.maximum(p_i - q, 0.0)
                    z = float(np.sum(res))
                    shift, mass = shift + mass, mass * z
                    if mass <= WSUM_FLOOR:
                        small_mass = True
                    if z <= 0.0:
                        p_i = None
                        break
                    p_i = res / z
                if nxt is None:
                    residual[b] = p_i is not None
                    w = p_i if p_i is not None else Pt[cur]
                    wsum[b] = mass if p_i is not None else 1.0
                    break
                path.append(nxt)
                cur = nxt
        out_accept[b] = acc.astype(np.uint8)
        y, m1, m2 = race_draw(w, seed, b, cur, offset, chunk)

        k = len(path)
        for j, c in enumerate(path[1:]):
            out_tokens[b, j] = tok[b, c]
        out_tokens[b, k - 1] = y
        out_path[b, :k] = path
        out_count[b] = k
        stop_row[b] = cur
        margin1[b], margin2[b] = m1, m2
        exempt[b] = (near_tie or small_mass or m1 <= 1.0 + RACE_MARGIN
                     or m2 <= 1.0 + RACE_MARGIN or (residual[b] and wsum[b] <= WSUM_FLOOR))

    return {
        "out_tokens": out_tokens, "out_count": out_count, "out_path": out_path,
        "out_accept": out_accept, "ratio": ratio_all, "u": u_all,
        "stop_row": stop_row, "residual": residual, "wsum": wsum,
        "margin1": margin1, "margin2": margin2, "exempt": exempt,
    }
