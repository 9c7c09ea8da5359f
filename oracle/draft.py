"""fp64 draft-step token draw -- test infrastructure (oracle side).

"Guide to MagicDec", step 2 of its reference implementation (the drafter):
at each draft step the draft model's logits for the next position go
through a softmax, one token is drawn from the resulting distribution, and
the distribution is kept for the verifier.

Readings taken where the page leaves a step open (each listed in the design
notes of the repository):

* the draw is an exponential race over p = softmax(l): id x gets
  E_x = -ln U_x with U_x = U(philox(x // 4, node, b, 4*offset + 1), word
  x % 4), scores p_x / E_x, and the largest score wins (ties: lowest id).
  Minimum-of-exponentials makes the winner x with probability p_x exactly,
  so this is a multinomial draw of one sample;
* ``node`` is the id of the node whose token is drawn (chain: draft step j
  draws node j + 1); stream 4*offset + 1 is the one spec_sample leaves free
  (it uses 4*offset + 0, 2, 3);
* the returned log-probability is ln p_x at the drawn id.
"""

from __future__ import annotations

import numpy as np

from .sample import softmax, uniforms

STREAM_DRAFT = 1
DRAFT_MARGIN = 1e-9   # best/second race score at or below 1 + this is a near-tie


def draft_sample(logits, seed: int, offset: int, node: int):
    """Draw one token per row of ``logits`` [B, V].

    Returns dict(token [B] int32, logprob [B] float64, margin [B] float64,
    exempt [B] bool) where margin is the ratio of the two best race scores.
    """
    if hasattr(logits, "detach"):
        logits = logits.detach().to("cpu").double().numpy()
    lg = np.asarray(logits, dtype=np.float64)
    B, V = lg.shape
    token = np.full(B, -1, dtype=np.int32)
    logprob = np.full(B, np.nan)
    margin = np.full(B, np.inf)
    ids = np.arange(V)
    for b in range(B):
        if not np.isfinite(lg[b]).any():
            continue
        p = softmax(lg[b])
        u = uniforms(seed, ids // 4, node, b, 4 * offset + STREAM_DRAFT, ids % 4)
        score = p / (-np.log(u))
        x = int(np.argmax(score))           # first maximum: lowest id on ties
        token[b] = x
        logprob[b] = np.log(p[x])
        if V > 1:
            top2 = np.partition(score, V - 2)[V - 2:]
            with np.errstate(over="ignore"):
                margin[b] = top2[1] / top2[0] if top2[0] > 0 else np.inf
    return {"token": token, "logprob": logprob, "margin": margin,
            "exempt": margin <= 1.0 + DRAFT_MARGIN}
