"""GPU parity of spec_window_attention (draft window + sinks) against the fp64 oracle."""

import numpy as np
import pytest
import torch

from oracle.attention import window_attention as oracle_window
from tests.gpu_util import assert_attention_close, say
from workloads import make_window_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(x, B, Hq, Hkv, D, W, S, fused=False, num_splits=0):
    import long_context_verify_amd as L
    out, lse = L.window_attention(x["q"], x["k_ring"], x["v_ring"], x["k_sink"], x["v_sink"],
                                  x["total_len"], k_new=x["k_new"] if fused else None,
                                  v_new=x["v_new"] if fused else None, num_splits=num_splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_window(x["q"], x["hist_sink_k"], x["hist_sink_v"], x["hist_recent_k"],
                                 x["hist_recent_v"], x["total_len"], W, S)
    return out, lse, o_ref, l_ref


CASES = [
    # name, B, Hq, Hkv, D, W, S, T list, dtype
    ("tiny_fp32_w128", 1, 8, 2, 64, 128, 4, [1024], "f32"),
    ("llama8b_w512_bf16", 8, 32, 8, 128, 512, 4, [32768] * 8, "bf16"),
    ("magicdec_w256_bf16", 4, 32, 8, 128, 256, 4, [131072] * 4, "bf16"),
    ("mixed_T_bf16", 6, 8, 2, 128, 64, 4, [1, 3, 4, 5, 68, 200], "bf16"),
    ("mixed_T_fp32", 6, 8, 2, 128, 64, 4, [1, 2, 4, 67, 68, 300], "f32"),
    ("no_sinks_bf16", 2, 8, 2, 64, 96, 0, [50, 1000], "bf16"),
    ("wrap_4W_bf16", 3, 16, 4, 128, 40, 4, [4 * 40 + 1, 4 * 40 + 4, 161 + 39], "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_parity(case):
    name, B, Hq, Hkv, D, W, S, T, dt = case
    say(f"window {name}")
    x = make_window_inputs(B, Hq, Hkv, D, W, S, T, dtype=dt, seed=sum(map(ord, name)), device=DEV)
    out, lse, o_ref, l_ref = _run(x, B, Hq, Hkv, D, W, S)
    assert_attention_close(out, lse, o_ref, l_ref, x["q"].dtype, name)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_window_fused_append(dt):
    B, Hq, Hkv, D, W, S = 5, 8, 2, 128, 48, 4
    T = [1, 4, 5, 52, 300]           # new token in a sink slot, first ring slot, and wrapped ring
    say(f"window fused append {dt}")
    x = make_window_inputs(B, Hq, Hkv, D, W, S, T, dtype=dt, seed=31, device=DEV,
                           fused_append=True)
    out, lse, o_ref, l_ref = _run(x, B, Hq, Hkv, D, W, S, fused=True)
    assert_attention_close(out, lse, o_ref, l_ref, x["q"].dtype, "fused append")
    for b, t in enumerate(T):        # the new token now sits in its slot
        if t - 1 < S:
            assert torch.equal(x["k_sink"][b, :, t - 1], x["k_new"][b, :, 0])
            assert torch.equal(x["v_sink"][b, :, t - 1], x["v_new"][b, :, 0])
        else:
            s = (t - 1 - S) % W
            assert torch.equal(x["k_ring"][b, :, s], x["k_new"][b, :, 0])
            assert torch.equal(x["v_ring"][b, :, s], x["v_new"][b, :, 0])


def test_window_equals_verify_attention_when_window_covers_history():
    """T <= S + W: the draft window sees every token, i.e. full attention of one query."""
    import long_context_verify_amd as L
    B, Hq, Hkv, D, W, S, T = 2, 8, 2, 128, 256, 4, 200
    say("window == full attention")
    x = make_window_inputs(B, Hq, Hkv, D, W, S, [T, T], dtype="bf16", seed=9, device=DEV)
    out, _ = L.window_attention(x["q"], x["k_ring"], x["v_ring"], x["k_sink"], x["v_sink"],
                                x["total_len"])
    k = torch.cat([x["hist_sink_k"], x["hist_recent_k"][:, :, W - (T - S):]], dim=2).contiguous()
    v = torch.cat([x["hist_sink_v"], x["hist_recent_v"][:, :, W - (T - S):]], dim=2).contiguous()
    full, _ = L.verify_attention(x["q"], k, v)
    torch.cuda.synchronize()
    assert (out.float() - full.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("splits", [1, 2, 5, 9, 17, 64])
def test_window_split_independence(splits):
    say(f"window splits={splits}")
    B, Hq, Hkv, D, W, S = 2, 32, 8, 128, 512, 4
    x = make_window_inputs(B, Hq, Hkv, D, W, S, [5000, 300], dtype="bf16", seed=splits, device=DEV)
    out, lse, o_ref, l_ref = _run(x, B, Hq, Hkv, D, W, S, num_splits=splits)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, f"splits={splits}")


@pytest.mark.parametrize("Hq,Hkv,D", [(64, 2, 128), (64, 2, 64), (16, 4, 64), (8, 8, 128)])
def test_window_split_merge_shapes(Hq, Hkv, D):
    """Every epilogue shape of the in-kernel split merge: 16- and 32-row query
    slices (g <= 16 and g = 32), head dim 64 and 128, three splits."""
    say(f"window merge shapes Hq={Hq} Hkv={Hkv} D={D}")
    B, W, S = 3, 200, 4
    x = make_window_inputs(B, Hq, Hkv, D, W, S, [1000, 150, 2], dtype="bf16",
                           seed=Hq * 1000 + Hkv * 10 + D, device=DEV)
    out, lse, o_ref, l_ref = _run(x, B, Hq, Hkv, D, W, S, num_splits=3)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, f"{Hq}/{Hkv}/{D}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("W,S", [(1, 0), (1, 4), (2, 1)])
def test_window_degenerate_sizes(dt, W, S):
    """A one- or two-slot ring, with and without sinks, from the first token
    to well past the wrap-around, plain and with the fused append."""
    name = f"W{W}_S{S}_{dt}"
    say(f"window degenerate {name}")
    T = [1, 2, 3, 5, 6, 37]
    x = make_window_inputs(len(T), 8, 2, 64, W, S, T, dtype=dt, seed=W * 10 + S, device=DEV)
    out, lse, o_ref, l_ref = _run(x, len(T), 8, 2, 64, W, S)
    assert_attention_close(out, lse, o_ref, l_ref, x["q"].dtype, name)
    x = make_window_inputs(len(T), 8, 2, 64, W, S, T, dtype=dt, seed=W * 10 + S + 1, device=DEV,
                           fused_append=True)
    out, lse, o_ref, l_ref = _run(x, len(T), 8, 2, 64, W, S, fused=True)
    assert_attention_close(out, lse, o_ref, l_ref, x["q"].dtype, name + " fused")


def test_window_wide_ring():
    """A 4096-slot ring (129 chunks: many splits per unit) at 100K tokens."""
    say("window W=4096")
    B, Hq, Hkv, D, W, S = 2, 32, 8, 128, 4096, 4
    x = make_window_inputs(B, Hq, Hkv, D, W, S, [100000, 2000], dtype="bf16", seed=4096,
                           device=DEV)
    out, lse, o_ref, l_ref = _run(x, B, Hq, Hkv, D, W, S)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, "W=4096")


def test_window_bad_total_len_flags_error():
    import long_context_verify_amd as L
    say("window total_len 0")
    x = make_window_inputs(2, 8, 2, 64, 32, 4, [10, 10], dtype="bf16", seed=2, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    tl = torch.tensor([10, 0], dtype=torch.int32, device=DEV)
    out, lse = L.window_attention(x["q"], x["k_ring"], x["v_ring"], x["k_sink"], x["v_sink"], tl,
                                  dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 0x4
    assert torch.all(out[1] == 0)


@pytest.mark.parametrize("dt,tol", [("f32", 1e-6), ("bf16", 8e-3)])
def test_window_full_ring_rotation_invariance(dt, tol):
    """With a full ring every slot is attended, so rotating the slots (a permutation
    of the keys) leaves the output unchanged up to summation order."""
    import long_context_verify_amd as L
    say(f"window ring rotation {dt}")
    B, Hq, Hkv, D, W, S = 3, 16, 4, 128, 96, 4
    x = make_window_inputs(B, Hq, Hkv, D, W, S, [S + W + 7, 1000, 5 * W], dtype=dt, seed=21,
                           device=DEV)
    out, lse = L.window_attention(x["q"], x["k_ring"], x["v_ring"], x["k_sink"], x["v_sink"],
                                  x["total_len"])
    kr = torch.roll(x["k_ring"], shifts=37, dims=2).contiguous()
    vr = torch.roll(x["v_ring"], shifts=37, dims=2).contiguous()
    out2, lse2 = L.window_attention(x["q"], kr, vr, x["k_sink"], x["v_sink"], x["total_len"])
    torch.cuda.synchronize()
    assert (out.float() - out2.float()).abs().max().item() <= tol
    assert (lse - lse2).abs().max().item() <= 1e-5


@pytest.mark.parametrize("dt,splits,tol", [("f32", 0, 1e-5), ("bf16", 0, 1e-4), ("bf16", 3, 1e-4)])
def test_window_constant_keys_count_the_attended_tokens(dt, splits, tol):
    """Equal keys: lse - score = ln(min(S, T) + min(W, T - S)) on the GPU too
    (bf16: MFMA kernel, whose splits merge in the last work-group)."""
    import long_context_verify_amd as L
    say(f"window constant keys {dt} splits={splits}")
    W, S, D = 64, 4, 128
    Ts = [1, 3, 4, 5, 40, 68, 69, 500]
    B = len(Ts)
    x = make_window_inputs(B, 8, 2, D, W, S, Ts, dtype=dt, seed=5, device=DEV)
    x["k_ring"][:] = 0.125
    x["k_sink"][:] = 0.125
    _, lse = L.window_attention(x["q"], x["k_ring"], x["v_ring"], x["k_sink"], x["v_sink"],
                                x["total_len"], num_splits=splits)
    torch.cuda.synchronize()
    s = (x["q"][:, :, 0].double() * 0.125).sum(-1) / np.sqrt(D)
    counts = torch.tensor([min(S, T) + min(W, max(T - S, 0)) for T in Ts], dtype=torch.float64,
                          device=DEV)
    err = (lse[:, :, 0].double() - s - torch.log(counts)[:, None]).abs().max().item()
    assert err <= tol
