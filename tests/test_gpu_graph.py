"""The hot path inside a captured HIP graph.

The kernels allocate nothing, issue no memsets and leave their workspace
arrival counters at zero, so one verify + window + sampling step can be
captured once and replayed.  Each replay runs on fresh inputs copied in
place (eager work between replays) and must equal, bit for bit, the same
calls made eagerly on those inputs with their own buffers.
"""

import pytest
import torch

from tests.gpu_util import say
from workloads import make_attention_inputs, make_sample_inputs, make_window_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_step_replays_match_eager_calls():
    import long_context_verify_amd as L
    say("graph capture of one step")
    B, Hq, Hkv, n_q, D, Lk = 4, 32, 8, 5, 128, 4096
    W, S, V = 256, 4, 50000
    bf16 = torch.bfloat16

    def fresh(i):
        x = make_attention_inputs(B, Hq, Hkv, n_q, D, Lk, dtype="bf16", seed=200 + i, device=DEV)
        w = make_window_inputs(B, Hq, Hkv, D, W, S, [5000, 77, 300, 261], dtype="bf16",
                               seed=300 + i, device=DEV)
        s = make_sample_inputs(B, n_q, V, None, 3.0, draft_noise_std=1.0, seed=400 + i,
                               device=DEV)
        return x, w, s

    # Static buffers the graph reads and writes.
    x, w, s = fresh(0)
    ws_v = torch.zeros(L.verify_attention_workspace_bytes(B, Hq, Hkv, n_q, D, Lk, bf16),
                       dtype=torch.uint8, device=DEV)
    ws_w = torch.zeros(L.window_attention_workspace_bytes(B, Hq, Hkv, D, W, S, bf16),
                       dtype=torch.uint8, device=DEV)
    ws_s = torch.zeros(L.sample_workspace_bytes(B, n_q, V), dtype=torch.uint8, device=DEV)
    out, lse = torch.empty_like(x["q"]), torch.empty(B, Hq, n_q, device=DEV)
    wout, wlse = torch.empty_like(w["q"]), torch.empty(B, Hq, 1, device=DEV)
    s_out = dict(out_tokens=torch.empty(B, n_q, dtype=torch.int32, device=DEV),
                 out_count=torch.empty(B, dtype=torch.int32, device=DEV),
                 out_path=torch.empty(B, n_q, dtype=torch.int32, device=DEV),
                 out_accept=torch.empty(B, n_q, dtype=torch.uint8, device=DEV))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)

    def step():
        L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"], out=out, lse=lse, workspace=ws_v,
                           dev_err=err)
        L.window_attention(w["q"], w["k_ring"], w["v_ring"], w["k_sink"], w["v_sink"],
                           w["total_len"], out=wout, lse=wlse, workspace=ws_w, dev_err=err)
        L.spec_sample(s["target"], s["draft"], s["tokens"], seed=7, offset=3, workspace=ws_s,
                      dev_err=err, **s_out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    for rep in range(1, 5):
        nx, nw, ns = fresh(rep)
        for src, dst in ((nx, x), (nw, w), (ns, s)):
            for k in dst:
                if isinstance(dst[k], torch.Tensor):
                    dst[k].copy_(src[k])
        g.replay()
        torch.cuda.synchronize()
        e_out, e_lse = L.verify_attention(nx["q"], nx["k"], nx["v"], nx["kv_len"])
        e_wout, e_wlse = L.window_attention(nw["q"], nw["k_ring"], nw["v_ring"], nw["k_sink"],
                                            nw["v_sink"], nw["total_len"])
        e_s = L.spec_sample(ns["target"], ns["draft"], ns["tokens"], seed=7, offset=3)
        torch.cuda.synchronize()
        assert torch.equal(out, e_out) and torch.equal(lse, e_lse), f"replay {rep}: verify"
        assert torch.equal(wout, e_wout) and torch.equal(wlse, e_wlse), f"replay {rep}: window"
        for k in s_out:
            assert torch.equal(s_out[k], e_s[k]), f"replay {rep}: {k}"
    assert int(err.item()) == 0
