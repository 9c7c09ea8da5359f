"""Bit stability of every kernel that hands partials from one work-group to
another in the same launch (the last work-group of a group to arrive reads
the others' partials and finishes the group): the draft window's split
merge, the sampling draw and the draft-step draw.  The verify chain kernel's
merge has its own test in test_gpu_attention.py.

The handoff orders device-scope stores and loads with per-thread waits and a
relaxed arrival counter (no release/acquire fences), so it rests on the
hardware's ordering of those accesses.  Here two different inputs alternate
for 24 calls on ONE workspace, at sizes with hundreds of work-groups
arriving per group: every call must reproduce, bit for bit, the first call on
the same input (a partial read before it landed, or one left over from the
other input, would change a result), no error bit may be set, and the
arrival counters must be back at zero afterwards."""

import numpy as np
import pytest
import torch

from tests.gpu_util import say
from workloads import make_sample_inputs, make_window_inputs, random_tree

pytestmark = pytest.mark.gpu
DEV = "cuda"
CALLS = 24


def _lib():
    import long_context_verify_amd as L
    return L


def test_window_merge_interleaved_bit_stable():
    say("handoff: window split merge, 24 alternating calls")
    L = _lib()
    B, Hq, Hkv, D, W, S = 8, 32, 8, 128, 512, 4
    xs = [make_window_inputs(B, Hq, Hkv, D, W, S, [W + S + 977 * (i + 1)] * B, dtype="bf16",
                             seed=401 + i, device=DEV) for i in range(2)]
    splits = 9
    ws = torch.zeros(L.window_attention_workspace_bytes(B, Hq, Hkv, D, W, S, torch.bfloat16,
                                                        splits), dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = [L.window_attention(x["q"], x["k_ring"], x["v_ring"], x["k_sink"], x["v_sink"],
                               x["total_len"], num_splits=splits, workspace=ws, dev_err=err)
            for _ in range(CALLS // 2) for x in xs]
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for i, (o, l) in enumerate(outs):
        o0, l0 = outs[i % 2]
        assert torch.equal(o, o0) and torch.equal(l, l0), f"call {i}"
    assert not torch.equal(outs[0][0], outs[1][0])
    n_ctr = B * Hkv  # one arrival counter per (sequence, kv head) at the workspace's start
    assert int(ws[:4 * n_ctr].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("rule,tree", [("first", False), ("first", True), ("lossless", True)])
def test_sampling_draw_interleaved_bit_stable(rule, tree):
    say(f"handoff: sampling draw ({rule}, {'tree' if tree else 'chain'}), 24 alternating calls")
    L = _lib()
    B, V = 16, 128256
    N = 16 if tree else 5
    parent = random_tree(N, max_depth=4, max_children=3, seed=77) if tree else None
    par_t = None if parent is None else torch.as_tensor(parent, dtype=torch.int32, device=DEV)
    xs = [make_sample_inputs(B, N, V, parent, 3.0, draft_noise_std=1.0, seed=500 + i, device=DEV)
          for i in range(2)]
    ws = torch.zeros(L.sample_workspace_bytes(B, N, V), dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = []
    for k in range(CALLS):
        x = xs[k % 2]
        outs.append(L.spec_sample(x["target"], x["draft"], x["tokens"], parent=par_t, seed=9,
                                  offset=3, workspace=ws, dev_err=err, siblings=rule))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for i, o in enumerate(outs):
        o0 = outs[i % 2]
        for key in ("out_tokens", "out_count", "out_path", "out_accept"):
            assert torch.equal(o[key], o0[key]), f"call {i}: {key}"
    assert not torch.equal(outs[0]["out_tokens"], outs[1]["out_tokens"])
    # The arrival counters (the workspace's first region) are back at zero.
    assert int(ws[:B * 1088].view(torch.int32).abs().sum().item()) == 0


def test_draft_draw_interleaved_bit_stable():
    say("handoff: draft-step draw, 24 alternating calls")
    L = _lib()
    B, V = 64, 128256
    g = torch.Generator(device="cpu").manual_seed(606)
    xs = [(torch.randn(B, V, generator=g) * 3.0).to(DEV) for _ in range(2)]
    ws = torch.zeros(max(L.draft_sample_workspace_bytes(B, V), 256), dtype=torch.uint8,
                     device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = [L.draft_sample(xs[k % 2], 1, seed=11, offset=5, workspace=ws, dev_err=err)
            for k in range(CALLS)]
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for i, (tok, lp) in enumerate(outs):
        t0, l0 = outs[i % 2]
        assert torch.equal(tok, t0) and torch.equal(lp, l0), f"call {i}"
    assert not torch.equal(outs[0][0], outs[1][0])
