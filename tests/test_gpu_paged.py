"""GPU parity of spec_verify_attention_paged against the fp64 oracle.

Same tolerances as the contiguous verify path (max abs 1e-5 fp32 / 2e-2 bf16
on outputs, lse 1e-5 / 1e-2).  The page pool is a seeded shuffle of the
contiguous cache, with table entries past each sequence's pages set to -1 and
spare pages full of junk, so a read outside the table would show.  With the
same split count the paged and contiguous kernels do the same arithmetic, so
their outputs are also compared bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle.attention import verify_attention_paged as oracle_paged
from tests.gpu_util import assert_attention_close, say
from workloads import CONFIGS, make_attention_inputs, make_paged_inputs, random_tree

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _lib():
    import long_context_verify_amd as L
    return L


CASES = [
    # name, B, Hq, Hkv, n_q, D, L_cap, kv_len, dtype, P, tree, splits
    ("bf16_chain_p64", 3, 32, 8, 5, 128, 3000, [3000, 1234, 5], "bf16", 64, False, 0),
    ("bf16_chain_p256_split7", 2, 16, 4, 5, 128, 2600, [2600, 2555], "bf16", 256, False, 7),
    ("bf16_d64_nq3", 2, 16, 4, 3, 64, 1500, [1500, 700], "bf16", 128, False, 0),
    ("bf16_tree64_p64", 2, 32, 8, 64, 128, 1100, [1100, 900], "bf16", 64, True, 0),
    ("bf16_tree64_p128_split3", 2, 8, 2, 64, 128, 1300, [1300, 1234], "bf16", 128, True, 3),
    ("fp32_chain_p64", 2, 8, 2, 5, 64, 700, [700, 333], "f32", 64, False, 0),
    ("fp32_tree12_p64", 2, 8, 2, 12, 128, 400, [400, 130], "f32", 64, True, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_parity(case):
    name, B, Hq, Hkv, n_q, D, L_cap, kv, dt, P, tree, splits = case
    say(f"verify paged {name}")
    L = _lib()
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, L_cap, dtype=dt, seed=sum(map(ord, name)),
                              device=DEV, kv_len=kv)
    parent = random_tree(n_q, seed=7) if tree else None
    pg = make_paged_inputs(x["k"], x["v"], x["kv_len"], P, seed=5)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, lse = L.verify_attention_paged(x["q"], pg["k_pages"], pg["v_pages"], pg["block_table"],
                                        x["kv_len"], L_cap, parent=parent, num_splits=splits,
                                        dev_err=err)
    ref_out, ref_lse = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"], parent=parent,
                                          num_splits=splits)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    o_ref, l_ref = oracle_paged(x["q"].cpu(), pg["k_pages"].cpu(), pg["v_pages"].cpu(),
                                pg["block_table"].cpu(), x["kv_len"].cpu(), L_cap,
                                parent=None if parent is None else np.asarray(parent))
    assert_attention_close(out, lse, o_ref, l_ref, x["q"].dtype, name)
    # Short sequences: the paged plan equals the contiguous one, so the bits match.
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_paged_split_floor_for_long_sequences():
    """One split asked for, 40 000 keys at P = 64: the plan raises the split count so
    each split's page ids fit in LDS; the result is unchanged."""
    say("verify paged split floor")
    L = _lib()
    B, Hq, Hkv, n_q, D, Lc = 1, 8, 2, 5, 128, 40000
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, Lc, dtype="bf16", seed=12, device=DEV)
    pg = make_paged_inputs(x["k"], x["v"], x["kv_len"], 64, seed=2)
    out, lse = L.verify_attention_paged(x["q"], pg["k_pages"], pg["v_pages"], pg["block_table"],
                                        x["kv_len"], Lc, num_splits=1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_paged(x["q"].cpu(), pg["k_pages"].cpu(), pg["v_pages"].cpu(),
                                pg["block_table"].cpu(), x["kv_len"].cpu(), Lc)
    assert_attention_close(out, lse, o_ref, l_ref, torch.bfloat16, "split floor")


def test_paged_bad_page_sets_error_and_stays_finite():
    say("verify paged bad page id")
    L = _lib()
    B, Hq, Hkv, n_q, D, Lc = 2, 8, 2, 5, 128, 1000
    x = make_attention_inputs(B, Hq, Hkv, n_q, D, Lc, dtype="bf16", seed=13, device=DEV)
    pg = make_paged_inputs(x["k"], x["v"], x["kv_len"], 64, seed=3)
    bt = pg["block_table"].clone()
    bt[1, 3] = pg["k_pages"].shape[0] + 7     # outside the pool
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, lse = L.verify_attention_paged(x["q"], pg["k_pages"], pg["v_pages"], bt, x["kv_len"], Lc,
                                        dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0x40
    assert torch.isfinite(out.float()).all()
    o_ref, l_ref = oracle_paged(x["q"][:1].cpu(), pg["k_pages"].cpu(), pg["v_pages"].cpu(),
                                pg["block_table"][:1].cpu(), x["kv_len"][:1].cpu(), Lc)
    assert_attention_close(out[:1], lse[:1], o_ref, l_ref, torch.bfloat16, "good sequence")


@pytest.mark.parametrize("name", ["llama8b_32k_chain", "medusa_tree64_8k"])
def test_paged_full_size(name):
    """Whole workload through a shuffled 64-key page pool: bit-identical to the contiguous
    call with the same split count, and the oracle on sampled units."""
    cfg = CONFIGS[name]
    say(f"verify paged full-size {name}")
    L = _lib()
    x = make_attention_inputs(cfg.batch, cfg.hq, cfg.hkv, cfg.n_q, cfg.head_dim, cfg.kv_len,
                              dtype=cfg.dtype, seed=cfg.seed, device=DEV)
    parent = random_tree(cfg.n_q) if cfg.tree else None
    pg = make_paged_inputs(x["k"], x["v"], x["kv_len"], 64, seed=cfg.seed)
    splits = L.verify_attention_auto_splits(cfg.batch, cfg.hq, cfg.hkv, cfg.n_q, cfg.head_dim,
                                            cfg.kv_len, x["q"].dtype)
    out, lse = L.verify_attention_paged(x["q"], pg["k_pages"], pg["v_pages"], pg["block_table"],
                                        x["kv_len"], cfg.kv_len, parent=parent, num_splits=splits)
    ref_out, ref_lse = L.verify_attention(x["q"], x["k"], x["v"], x["kv_len"], parent=parent,
                                          num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    g = cfg.hq // cfg.hkv
    kp, vp = pg["k_pages"].cpu(), pg["v_pages"].cpu()
    bt, kl, q = pg["block_table"].cpu(), x["kv_len"].cpu(), x["q"].cpu()
    for b, hk in [(0, 0), (cfg.batch - 1, cfg.hkv - 1)]:
        sl = slice(hk * g, (hk + 1) * g)
        heads = [(0, h) for h in range(hk * g, (hk + 1) * g)]
        o_ref, l_ref = oracle_paged(q[b:b + 1], kp, vp, bt[b:b + 1], kl[b:b + 1], cfg.kv_len,
                                    parent=parent, heads=heads)
        assert_attention_close(out[b:b + 1, sl], lse[b:b + 1, sl], o_ref[:, sl], l_ref[:, sl],
                               torch.bfloat16, f"{name} unit {(b, hk)}")
