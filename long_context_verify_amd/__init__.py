"""MI355X-native (gfx950) kernels for the verification step of speculative decoding.

The computation lives in ``libspecverify.so`` (hand-written HIP, built from
``csrc/`` by ``build.py``) behind the C ABI of ``include/spec_verify.h``:

* ``verify_attention`` -- block-of-queries attention against the full KV
  cache, chain (causal) or candidate tree (ancestor-only) mask;
  ``verify_attention_paged`` reads the cache through a block table;
* ``window_attention`` -- the draft's bounded attention over sink tokens and
  a FIFO ring of the last W tokens, with an optional fused append;
* ``spec_sample`` -- vocabulary softmax, min(1, target/draft) acceptance and
  the residual / bonus draw (``spec_sample_noalloc``: the same without a
  workspace, for callers that cannot allocate);
* ``draft_sample`` -- one draft-step token draw from softmax(draft logits);
* ``kv_commit`` -- after sampling, keep the accepted path's K/V right after
  the prefix, set the new lengths, and rewind the draft ring.

This package only marshals torch tensors into those calls.
"""

from .api import (  # noqa: F401
    SPEC_BF16,
    SPEC_F32,
    SpecError,
    draft_sample,
    draft_sample_workspace_bytes,
    kv_commit,
    lib,
    sample_workspace_bytes,
    spec_sample,
    spec_sample_noalloc,
    status_str,
    validate_tree,
    verify_attention,
    verify_attention_auto_splits,
    verify_attention_paged,
    verify_attention_paged_workspace_bytes,
    verify_attention_workspace_bytes,
    window_attention,
    window_attention_workspace_bytes,
)

__all__ = [
    "SPEC_BF16", "SPEC_F32", "SpecError", "draft_sample", "draft_sample_workspace_bytes",
    "kv_commit", "lib", "sample_workspace_bytes", "spec_sample", "spec_sample_noalloc",
    "status_str", "validate_tree", "verify_attention", "verify_attention_auto_splits",
    "verify_attention_paged", "verify_attention_paged_workspace_bytes",
    "verify_attention_workspace_bytes", "window_attention", "window_attention_workspace_bytes",
]
