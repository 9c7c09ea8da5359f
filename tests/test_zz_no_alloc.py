"""spec_sample_noalloc (no workspace, library-owned scratch) against spec_sample.

The no-allocation entry point runs the same kernels as spec_sample_ex on the
library's per-device scratch array instead of a caller workspace, so on the
same inputs and Philox seed its outputs must equal spec_sample's bit for bit
(the sampling bar: tokens, counts, paths and accept flags exact).  Calls run
back to back on the shared array, each smaller than the one before, so a
result that depended on what an earlier call left in the array would show.
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import say
from workloads import make_sample_inputs, random_tree

pytestmark = pytest.mark.gpu
DEV = "cuda"

# name, B, N, V, tree, logits dtype, siblings
CALLS = [
    ("b64_chain_v128256", 64, 4, 128256, False, torch.float32, "first"),
    ("b8_chain_v32000", 8, 5, 32000, False, torch.float32, "first"),
    ("b4_tree16_v5001_bf16_lossless", 4, 16, 5001, True, torch.bfloat16, "lossless"),
    ("b1_single_node_v1000", 1, 1, 1000, False, torch.float32, "first"),
]


def _inputs(name, B, N, V, tree, dtype):
    parent = random_tree(N, max_depth=4, max_children=3, seed=5) if tree else None
    x = make_sample_inputs(B, N, V, parent, 3.0, draft_noise_std=1.0,
                           seed=sum(map(ord, name)), device=DEV)
    if dtype == torch.bfloat16:
        x["target"] = x["target"].to(torch.bfloat16)
        x["draft"] = x["draft"].to(torch.bfloat16)
    return x, parent


def _run(fn, x, parent, seed, offset, siblings):
    r = fn(x["target"], x["draft"], x["tokens"], parent=parent, seed=seed, offset=offset,
           siblings=siblings)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items()}


def test_noalloc_matches_spec_sample_on_successive_calls():
    import long_context_verify_amd as L
    for rep in range(2):
        for name, B, N, V, tree, dtype, sib in CALLS:
            say(f"noalloc {name} rep {rep}")
            x, parent = _inputs(name, B, N, V, tree, dtype)
            seed, offset = 0x5EED0000 + rep, 3 + rep
            dev_err = torch.zeros(1, dtype=torch.int32, device=DEV)
            got = L.spec_sample_noalloc(x["target"], x["draft"], x["tokens"], parent=parent,
                                        seed=seed, offset=offset, siblings=sib, dev_err=dev_err)
            torch.cuda.synchronize()
            got = {k: v.cpu().numpy() for k, v in got.items()}
            assert int(dev_err.item()) == 0, f"{name}: device error bits {int(dev_err.item())}"
            want = _run(L.spec_sample, x, parent, seed, offset, sib)
            for key in ("out_tokens", "out_count", "out_path", "out_accept"):
                assert np.array_equal(got[key], want[key]), f"{name} rep {rep}: {key} differs"


def test_noalloc_refuses_sizes_beyond_its_scratch():
    import long_context_verify_amd as L
    # 4096 sequences: their arrival counters alone exceed the 4 MiB array.
    assert L.sample_workspace_bytes(4096, 2, 1000) > 4 << 20
    t = torch.zeros(4096, 2, 1000, device=DEV)
    with pytest.raises(L.SpecError, match="UNSUPPORTED"):
        L.spec_sample_noalloc(t, t, torch.zeros(4096, 2, dtype=torch.int32, device=DEV))
