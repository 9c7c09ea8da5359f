"""GPU parity of spec_verify_attention against the fp64 oracle (MI355X).

Tolerances (max abs): 1e-5 for fp32 inputs, 2e-2 for bf16 inputs on the
outputs; lse 1e-5 / 1e-2; bf16 also holds a 1e-2 relative Frobenius error.
"""

import numpy as np
import pytest
import torch

from oracle.attention import verify_attention as oracle_verify
from tests.gpu_util import assert_attention_close, oracle_unit, say
from workloads import CONFIGS, make_attention_inputs, random_tree

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _lib():
    import long_context_verify_amd as L
    return L


def _gpu_and_oracle(x, parent=None, num_splits=0, scale=0.0):
    L = _lib()
    out, lse = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"], parent=parent,
                                  num_splits=num_splits, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_verify(x["q"], x["k"], x["v"], x["kv_len"],
                                 None if parent is None else np.asarray(parent),
                                 scale=scale if scale > 0 else None)
    return out, lse, o_ref, l_ref


CASES = [
    # name, B, Hq, Hkv, n_q, D, L, dtype, L_cap, kv_len
    ("tiny_chain_fp32", 1, 8, 2, 5, 64, 1024, "f32", None, None),
    ("fp32_d128_ragged", 3, 4, 2, 5, 128, 700, "f32", 777, [700, 5, 777]),
    ("bf16_chain_g4", 2, 32, 8, 5, 128, 4133, "bf16", None, None),
    ("bf16_chain_g1_M6", 2, 8, 8, 6, 128, 1000, "bf16", None, None),
    ("bf16_d64", 2, 16, 4, 4, 64, 2000, "bf16", 2100, [2000, 1999]),
    ("bf16_g8_M32", 1, 64, 8, 4, 128, 3000, "bf16", None, None),
    ("bf16_nq1", 2, 8, 2, 1, 128, 513, "bf16", None, None),
    ("bf16_only_block", 2, 8, 2, 5, 128, 5, "bf16", None, None),
    ("fp32_only_block", 1, 4, 1, 3, 64, 3, "f32", None, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chain_parity(case):
    name, B, Hq, Hkv, n_q, D, L, dt, L_cap, kv_len = case
    say(f"verify chain {name}")
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, L, dtype=dt, seed=sum(map(ord, name)),
                              device=DEV, L_cap=L_cap, kv_len=kv_len)
    out, lse, o_ref, l_ref = _gpu_and_oracle(x)
    assert_attention_close(out, lse, o_ref, l_ref, x["q"].dtype, name)


@pytest.mark.parametrize("splits", [1, 3, 7, 64, 1000])
def test_split_count_independence(splits):
    say(f"verify splits={splits}")
    x = make_attention_inputs(2, 16, 4, 5, 128, 3000, dtype="bf16", seed=splits, device=DEV)
    out, lse, o_ref, l_ref = _gpu_and_oracle(x, num_splits=splits)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, f"splits={splits}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_tree_parity(dt):
    say(f"verify tree 64 nodes {dt}")
    parent = random_tree(64, seed=4321)
    x = make_attention_inputs(2, 32, 8, 64, 128, 1024 + 64, dtype=dt, seed=77, device=DEV)
    out, lse, o_ref, l_ref = _gpu_and_oracle(x, parent=parent)
    assert_attention_close(out, lse, o_ref, l_ref, x["q"].dtype, f"tree {dt}")


@pytest.mark.parametrize("Hq,Hkv,n_q,D", [(64, 2, 1, 128), (32, 8, 4, 64), (64, 8, 4, 64),
                                           (16, 16, 3, 128)])
def test_chain_split_merge_shapes(Hq, Hkv, n_q, D):
    """The chain kernel's in-kernel split merge at every epilogue shape:
    16- and 32-row slices, head dim 64 and 128, several splits."""
    say(f"verify merge shapes Hq={Hq} Hkv={Hkv} n_q={n_q} D={D}")
    x = make_attention_inputs(2, Hq, Hkv, n_q, D, 2500, dtype="bf16", seed=Hq + n_q + D,
                              device=DEV, kv_len=[2500, 1111])
    out, lse, o_ref, l_ref = _gpu_and_oracle(x, num_splits=5)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, f"{Hq}/{Hkv}/{n_q}/{D}")


WIDE = [
    # name, B, Hq, Hkv, n_q, D, L, tree, splits, kv_len
    # two 256-row slices of the LDS-shared kernel (g = 8, 64 nodes)
    ("tree64_g8_two_slices", 2, 64, 8, 64, 128, 1500, True, 0, [1500, 700]),
    ("tree64_g8_two_slices_s3", 2, 64, 8, 64, 128, 1500, True, 3, [1500, 64]),
    # the longest chain (n_q = 64, g = 1): two live waves of the wide kernel
    ("chain_nq64_g1", 2, 8, 8, 64, 128, 2000, False, 0, [2000, 90]),
    # a wide block at D = 64 goes to the streaming kernel, eight 32-row slices
    ("tree64_d64_eight_slices", 2, 32, 8, 64, 64, 1200, True, 0, [1200, 333]),
    # a row count that leaves the last wave partly empty
    ("tree50_g4_M200", 3, 4, 1, 50, 128, 900, True, 2, [900, 50, 51]),
]


@pytest.mark.parametrize("case", WIDE, ids=[c[0] for c in WIDE])
def test_wide_query_blocks(case):
    """Query blocks at and past one wide slice: every row of every slice
    against the oracle, ragged lengths down to the block itself."""
    name, B, Hq, Hkv, n_q, D, L, tree, splits, kv_len = case
    say(f"verify wide {name}")
    parent = random_tree(n_q, seed=n_q + Hq) if tree else None
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, L, dtype="bf16", seed=sum(map(ord, name)),
                              device=DEV, kv_len=kv_len)
    out, lse, o_ref, l_ref = _gpu_and_oracle(x, parent=parent, num_splits=splits)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, name)


def test_tree_per_sequence_parent_and_forest():
    say("verify per-sequence parents incl. forest")
    n = 17
    parents = np.stack([random_tree(n, max_depth=3, max_children=3, seed=5),
                        np.full(n, -1, dtype=np.int32),
                        np.arange(-1, n - 1, dtype=np.int32)])
    x = make_attention_inputs(3, 8, 2, n, 128, 600, dtype="bf16", seed=8, device=DEV,
                              kv_len=[600, 300, 17])
    L = _lib()
    out, lse = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"], parent=parents)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_verify(x["q"], x["k"], x["v"], x["kv_len"], parents)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, "per-seq parents")


def test_chain_parent_array_matches_null_parent():
    say("verify explicit chain parent == NULL parent")
    x = make_attention_inputs(2, 32, 8, 5, 128, 2048, dtype="bf16", seed=3, device=DEV)
    L = _lib()
    o1, l1 = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"])
    o2, l2 = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"],
                                parent=np.arange(-1, 4, dtype=np.int32))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_needle_keys_move_the_running_max():
    """Keys equal to 4*q at a few positions shift the max between splits."""
    say("verify needle stress")
    B, Hq, Hkv, n_q, D, L = 1, 8, 2, 5, 128, 8192
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, L, dtype="bf16", seed=12, device=DEV)
    for pos in (17, 2500, 6000, L - n_q - 1):
        x["k"][0, :, pos] = (4.0 * x["q"][0, ::Hq // Hkv, 0].float()).to(torch.bfloat16)
    out, lse, o_ref, l_ref = _gpu_and_oracle(x, num_splits=9)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, "needle")


def test_custom_scale():
    say("verify custom scale")
    x = make_attention_inputs(1, 8, 2, 5, 128, 999, dtype="bf16", seed=4, device=DEV)
    out, lse, o_ref, l_ref = _gpu_and_oracle(x, scale=0.05)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, "scale")


def test_deterministic_bits():
    say("verify determinism")
    x = make_attention_inputs(4, 32, 8, 5, 128, 5000, dtype="bf16", seed=6, device=DEV)
    L = _lib()
    o1, l1 = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"])
    o2, l2 = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bad_kv_len_sets_error_and_zero_output():
    say("verify bad kv_len")
    x = make_attention_inputs(2, 8, 2, 5, 64, 100, dtype="bf16", seed=1, device=DEV,
                              kv_len=[100, 3])
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    L = _lib()
    out, lse = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"], dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 0x1
    assert torch.all(out[1] == 0)
    assert torch.all(torch.isneginf(lse[1]))
    o_ref, l_ref = oracle_verify(x["q"][:1], x["k"][:1], x["v"][:1], [100])
    assert_attention_close(out[:1], lse[:1], o_ref, l_ref, torch.bfloat16, "good sequence")


def test_workspace_reuse_across_calls():
    """The streaming kernel (chains, the draft window) merges its key-range
    splits in the work-group that finishes a unit last, counted in the
    workspace.  One zero-filled workspace serves a run of calls in turn
    (verify chains at several split counts, a tree, window calls) on inputs
    that change from round to round, so partials left by an earlier call
    would show: every result matches the oracle, no call reports an error,
    and the counters are back at zero afterwards."""
    from oracle.attention import window_attention as oracle_window
    from workloads import make_window_inputs
    say("verify workspace reuse")
    L = _lib()
    B, Hq, Hkv, D = 2, 16, 4, 128
    parent = random_tree(64, seed=12)
    nbytes = max([L.verify_attention_workspace_bytes(B, Hq, Hkv, 64, D, 3000, torch.bfloat16, s)
                  for s in (2, 3, 7, 16)] +
                 [L.window_attention_workspace_bytes(B, Hq, Hkv, D, 256, 4, torch.bfloat16, s)
                  for s in (0, 3)])
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    runs, wruns = [], []
    for rep in range(3):
        xs = [make_attention_inputs(B, Hq, Hkv, 5, D, 3000, dtype="bf16", seed=40 + rep,
                                    device=DEV),
              make_attention_inputs(B, Hq, Hkv, 64, D, 1500, dtype="bf16", seed=50 + rep,
                                    device=DEV)]
        for splits in (7, 3, 16):
            x = xs[0]
            runs.append((x, None, L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"],
                                                     num_splits=splits, workspace=ws,
                                                     dev_err=err)))
        x = xs[1]
        runs.append((x, parent, L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"],
                                                   parent=parent, num_splits=2 + rep,
                                                   workspace=ws, dev_err=err)))
        w = make_window_inputs(B, Hq, Hkv, D, 256, 4, [5000, 77 + rep], dtype="bf16",
                               seed=60 + rep, device=DEV)
        wruns.append((w, L.window_attention(w["q"], w["k_ring"], w["v_ring"], w["k_sink"],
                                            w["v_sink"], w["total_len"], num_splits=3,
                                            workspace=ws, dev_err=err)))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert int(ws[:256].count_nonzero().item()) == 0
    refs = {}
    for x, par, (out, lse) in runs:
        key = id(x)
        if key not in refs:
            refs[key] = oracle_verify(x["q"], x["k"], x["v"], x["kv_len"],
                                      None if par is None else np.asarray(par))
        assert_attention_close(out, lse, *refs[key], torch.bfloat16, "reused workspace")
    for w, wout in wruns:
        o_ref, l_ref = oracle_window(w["q"], w["hist_sink_k"], w["hist_sink_v"],
                                     w["hist_recent_k"], w["hist_recent_v"], w["total_len"], 256, 4)
        assert_attention_close(*wout, o_ref, l_ref, torch.bfloat16, "window, reused workspace")


def test_interleaved_calls_on_one_workspace_are_bit_stable():
    """Two inputs alternate for 24 calls on one workspace (the chain call
    merges its splits through it): every call reproduces, bit for bit, the
    result of the first call on the same input, so no partial of the other
    input is ever read."""
    say("verify interleaved calls on one workspace")
    L = _lib()
    B, Hq, Hkv, n_q, D, Lk = 4, 32, 8, 5, 128, 6000
    xs = [make_attention_inputs(B, Hq, Hkv, n_q, D, Lk, dtype="bf16", seed=90 + i, device=DEV)
          for i in range(2)]
    ws = torch.zeros(L.verify_attention_workspace_bytes(B, Hq, Hkv, n_q, D, Lk, torch.bfloat16, 6),
                     dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = [L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"], num_splits=6, workspace=ws,
                               dev_err=err) for x in xs * 12]
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for i, (o, l) in enumerate(outs):
        o0, l0 = outs[i % 2]
        assert torch.equal(o, o0) and torch.equal(l, l0), f"call {i}"
    assert not torch.equal(outs[0][0], outs[1][0])


def test_unzeroed_workspace_is_reported():
    """Arrival counters that were not zero-filled (the draft window, whose
    splits merge in the last work-group): the call sets SPEC_DEVERR_WORKSPACE
    and every kernel still runs to completion."""
    from workloads import make_window_inputs
    say("window unzeroed workspace")
    L = _lib()
    w = make_window_inputs(2, 16, 4, 128, 256, 4, [5000, 77], dtype="bf16", seed=3, device=DEV)
    nbytes = L.window_attention_workspace_bytes(2, 16, 4, 128, 256, 4, torch.bfloat16, 3)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    L.window_attention(w["q"], w["k_ring"], w["v_ring"], w["k_sink"], w["v_sink"],
                       w["total_len"], num_splits=3, workspace=ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0x80


@pytest.mark.parametrize("L,n_q,tree", [(262144, 5, False), (65536, 64, True)])
def test_longest_contexts(L, n_q, tree):
    """256K keys (a 512 MB unit stride, 32 splits per unit) and a 64-node tree
    at 64K, one sequence, ragged against the capacity: every unit against the
    oracle."""
    say(f"verify long context L={L} n_q={n_q}")
    B, Hq, Hkv, D = 1, 32, 8, 128
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, L - 123, dtype="bf16", seed=L % 997 + n_q,
                              device=DEV, L_cap=L)
    parent = random_tree(n_q, seed=64) if tree else None
    out, lse = _lib().verify_attention(x["q"], x["k"], x["v"], x["kv_len"], parent=parent)
    torch.cuda.synchronize()
    g = Hq // Hkv
    for hk in range(Hkv):
        o_ref, l_ref = oracle_unit(x["q"], x["k"], x["v"], x["kv_len"], parent, 0, hk, g)
        assert_attention_close(out[:, hk * g:(hk + 1) * g], lse[:, hk * g:(hk + 1) * g], o_ref,
                               l_ref, torch.bfloat16, f"L={L} unit {hk}")


FULL = ["llama8b_32k_chain", "magicdec_128k_chain", "medusa_tree64_8k", "llama70b_16k_chain_b64"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_units(name):
    """Whole workload on the GPU in the benchmarked launch shape; oracle on sampled units."""
    cfg = CONFIGS[name]
    say(f"verify full-size {name}")
    x = make_attention_inputs(cfg.batch, cfg.hq, cfg.hkv, cfg.n_q, cfg.head_dim, cfg.kv_len,
                              dtype=cfg.dtype, seed=cfg.seed, device=DEV)
    parent = random_tree(cfg.n_q) if cfg.tree else None
    L = _lib()
    out, lse = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"], parent=parent)
    torch.cuda.synchronize()
    g = cfg.hq // cfg.hkv
    rng = np.random.default_rng(cfg.seed)
    units = {(0, 0), (cfg.batch - 1, cfg.hkv - 1)}
    while len(units) < 4:
        units.add((int(rng.integers(cfg.batch)), int(rng.integers(cfg.hkv))))
    for b, hk in sorted(units):
        o_ref, l_ref = oracle_unit(x["q"], x["k"], x["v"], x["kv_len"], parent, b, hk, g)
        assert_attention_close(out[b:b + 1, hk * g:(hk + 1) * g], lse[b:b + 1, hk * g:(hk + 1) * g],
                               o_ref, l_ref, torch.bfloat16, f"{name} unit {(b, hk)}")
    assert torch.isfinite(out.float()).all()
