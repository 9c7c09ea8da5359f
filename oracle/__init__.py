"""fp64 CPU oracle of the speculative verification step -- TEST INFRASTRUCTURE.

Plain, slow, obviously-correct numpy definitions of what the GPU path
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here; the
product path (``long_context_verify_amd``) never does, and this package
imports nothing from it.  The two share no code: the only common source is
the seeded input generator in ``workloads/``, which holds none of the
method's arithmetic.

Contents and the passages they follow:

* ``attention.verify_attention`` -- attention of a block of query tokens
  (a gamma+1 causal chain or an N-node candidate tree under an
  ancestor-only mask) against the full KV cache.  "Guide to MagicDec",
  section "Lossless Target Model Verification Across Full Context";
  "Speculative Decoding in LLM Serving Systems", section "The algorithm",
  step 2 (Verify), and section "Tree-based variants" (Medusa: every token
  attends only to its tree ancestors).
* ``attention.window_attention`` -- one draft-step query against the S sink
  tokens plus the last W tokens.  "Guide to MagicDec", section "Fixed-Window
  KV Cache Decoupling" (bounded window, T_draft = O(W)) and "Best Practices",
  item 1 (attention-sink slots).
* ``sample.spec_sample`` -- softmax, acceptance test with min(1, target/draft),
  residual resample from the normalised max(target - draft, 0) or a bonus
  token from the last target row.  "Guide to MagicDec", section 2 (the
  acceptance and resampling equations); "Speculative Decoding & Medusa
  Architecture", section 2 (speculative sampling step); "Speculative
  Decoding in LLM Serving Systems", section "Accepting and rejecting".
* ``philox`` -- the Philox4x32-10 counter-based generator of Salmon, Moraes,
  Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11),
  written from the paper's definition; it supplies every uniform the
  sampler draws.

Parity status: every function above is pinned by ``-m "not gpu"`` tests
against library routines, closed forms, invariants or brute force.
"""


