"""GPU parity of spec_kv_commit against the oracle's commit (bit-exact).

Paths are root-to-node chains of seeded candidate trees (what the sampler's
walk returns).  Small cases compare whole caches and lengths; the full-size
tree and chain workloads compare the verified block region element by
element and check that every row before it is untouched.
"""

import numpy as np
import pytest
import torch

from oracle.attention import ancestors
from oracle.cache import commit_path, rollback_draft
from tests.gpu_util import say
from workloads import CONFIGS, chain_parent, random_tree

pytestmark = pytest.mark.gpu
DEV = "cuda"
ERR_KV_LEN, ERR_TOTAL_LEN, ERR_PATH = 0x1, 0x4, 0x10


def _paths(parent, B, n_q, rng, count0=()):
    """Random root-to-node paths (one per sequence), -1 padded; count 0 where asked."""
    path = np.full((B, n_q), -1, dtype=np.int32)
    count = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if b in count0:
            continue
        p = ancestors(parent, int(rng.integers(0, n_q)))[::-1]
        path[b, :len(p)] = p
        count[b] = len(p)
    return path, count


def _cache(B, Hkv, L_cap, D, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    k = torch.randn(B, Hkv, L_cap, D, generator=g, device=DEV).to(dtype)
    v = torch.randn(B, Hkv, L_cap, D, generator=g, device=DEV).to(dtype)
    return k, v


def _run(k, v, kv_len, count, n_q, path=None, total=None, appended=0):
    import long_context_verify_amd as L
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    L.kv_commit(k, v, kv_len, count, n_q, path=path, draft_total_len=total,
                draft_appended=appended, dev_err=err)
    torch.cuda.synchronize()
    return int(err.item())


SMALL = [
    # name, B, Hkv, n_q, D, L_cap, dtype, tree
    ("tree12_bf16_d128", 6, 2, 12, 128, 80, torch.bfloat16, True),
    ("tree64_bf16_d128", 5, 3, 64, 128, 200, torch.bfloat16, True),
    ("tree9_f32_d64", 4, 2, 9, 64, 40, torch.float32, True),
    ("chain5_f32_d64_path", 3, 2, 5, 64, 30, torch.float32, False),
    ("single_node", 3, 1, 1, 128, 9, torch.bfloat16, False),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_commit_small_whole_cache(case):
    name, B, Hkv, n_q, D, L_cap, dtype, tree = case
    say(f"kv_commit {name}")
    rng = np.random.default_rng(7)
    parent = random_tree(n_q, seed=31) if tree else chain_parent(n_q)
    path, count = _paths(parent, B, n_q, rng, count0=(1,) if B > 2 else ())
    kv_len = rng.integers(n_q, L_cap + 1, size=B).astype(np.int32)
    k, v = _cache(B, Hkv, L_cap, D, dtype, seed=3)
    k_ref, v_ref, L_ref = commit_path(k.cpu().float().numpy(), v.cpu().float().numpy(), kv_len,
                                      path, count, n_q)
    kl = torch.tensor(kv_len, device=DEV)
    err = _run(k, v, kl, torch.tensor(count, device=DEV), n_q, torch.tensor(path, device=DEV))
    assert err == 0
    assert kl.cpu().numpy().tolist() == L_ref.tolist()
    assert np.array_equal(k.cpu().float().numpy(), k_ref)
    assert np.array_equal(v.cpu().float().numpy(), v_ref)


def test_commit_chain_null_path_and_draft_rewind():
    say("kv_commit chain null path + draft rewind")
    B, Hkv, n_q, D, L_cap = 7, 2, 5, 128, 64
    rng = np.random.default_rng(2)
    count = np.array([1, 2, 3, 4, 5, 0, 5], dtype=np.int32)
    kv_len = rng.integers(n_q, L_cap + 1, size=B).astype(np.int32)
    total = rng.integers(20, 40, size=B).astype(np.int32)
    k, v = _cache(B, Hkv, L_cap, D, torch.bfloat16, seed=4)
    k0, v0 = k.clone(), v.clone()
    kl, tl = torch.tensor(kv_len, device=DEV), torch.tensor(total, device=DEV)
    err = _run(k, v, kl, torch.tensor(count, device=DEV), n_q, None, tl, appended=4)
    assert err == 0
    assert torch.equal(k, k0) and torch.equal(v, v0)
    path = np.tile(np.arange(n_q, dtype=np.int32), (B, 1))
    _, _, L_ref = commit_path(np.zeros((B, 1, L_cap, 1)), np.zeros((B, 1, L_cap, 1)), kv_len,
                              path, count, n_q)
    assert kl.cpu().numpy().tolist() == L_ref.tolist()
    assert tl.cpu().numpy().tolist() == rollback_draft(total, count, 4).tolist()


def test_commit_device_errors_leave_sequences_unchanged():
    say("kv_commit device-data errors")
    B, Hkv, n_q, D, L_cap = 5, 2, 6, 64, 32
    path = np.tile(np.arange(n_q, dtype=np.int32), (B, 1))
    path[0, :3] = [0, 2, 2]          # not strictly increasing
    path[1, :2] = [1, 2]             # does not start at the root
    path[3, :3] = [0, 3, 5]          # valid, moves rows
    count = np.array([3, 2, 2, 3, 7], dtype=np.int32)   # sequence 4: count > n_q
    kv_len = np.array([20, 20, 40, 20, 20], dtype=np.int32)  # sequence 2: beyond L_cap
    total = np.array([9, 9, 9, 9, 9], dtype=np.int32)
    k, v = _cache(B, Hkv, L_cap, D, torch.float32, seed=5)
    k_ref, v_ref, _ = commit_path(k.cpu().numpy(), v.cpu().numpy(), kv_len,
                                  np.where(np.arange(B)[:, None] == 3, path, -1),
                                  np.where(np.arange(B) == 3, count, 0), n_q)
    kl, tl = torch.tensor(kv_len, device=DEV), torch.tensor(total, device=DEV)
    err = _run(k, v, kl, torch.tensor(count, device=DEV), n_q, torch.tensor(path, device=DEV),
               tl, appended=5)
    assert err == ERR_PATH | ERR_KV_LEN
    assert kl.cpu().numpy().tolist() == [20, 20, 40, 17, 20]
    assert tl.cpu().numpy().tolist() == [9, 9, 9, 7, 9]
    assert np.array_equal(k.cpu().numpy(), k_ref) and np.array_equal(v.cpu().numpy(), v_ref)
    # A rewind below one token is refused for that sequence only.
    tl2 = torch.tensor([1, 9, 9, 9, 9], dtype=torch.int32, device=DEV)
    count2 = torch.tensor([1, 1, 1, 1, 1], dtype=torch.int32, device=DEV)
    kl2 = torch.tensor([20] * B, dtype=torch.int32, device=DEV)
    err = _run(k, v, kl2, count2, n_q, None, tl2, appended=2)
    assert err == ERR_TOTAL_LEN
    assert kl2.cpu().numpy().tolist() == [20, 15, 15, 15, 15]
    assert tl2.cpu().numpy().tolist() == [1, 8, 8, 8, 8]


@pytest.mark.parametrize("cfg", ["medusa_tree64_8k", "llama8b_32k_chain"])
def test_commit_full_size(cfg):
    c = CONFIGS[cfg]
    B, Hkv, n_q, D, L = c.batch, c.hkv, c.n_q, c.head_dim, c.kv_len
    say(f"kv_commit full size {cfg}")
    rng = np.random.default_rng(11)
    parent = random_tree(n_q) if c.tree else chain_parent(n_q)
    path, count = _paths(parent, B, n_q, rng)
    k, v = _cache(B, Hkv, L, D, torch.bfloat16, seed=6)
    p0 = L - n_q
    blk_k = k[:, :, p0:].float().cpu().numpy()
    blk_v = v[:, :, p0:].float().cpu().numpy()
    head_k, head_v = k[:, :, :p0].clone(), v[:, :, :p0].clone()
    ref_k, ref_v, _ = commit_path(blk_k, blk_v, np.full(B, n_q), path, count, n_q)
    kl = torch.full((B,), L, dtype=torch.int32, device=DEV)
    err = _run(k, v, kl, torch.tensor(count, device=DEV), n_q, torch.tensor(path, device=DEV))
    assert err == 0
    assert kl.cpu().numpy().tolist() == (p0 + count).tolist()
    assert np.array_equal(k[:, :, p0:].float().cpu().numpy(), ref_k)
    assert np.array_equal(v[:, :, p0:].float().cpu().numpy(), ref_v)
    assert torch.equal(k[:, :, :p0], head_k) and torch.equal(v[:, :, :p0], head_v)
