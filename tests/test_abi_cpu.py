"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every function include/spec_verify.h declares,
and reject bad arguments on the host before any HIP call (so these run on a
machine without a device).  Fake but aligned pointer values are used where a
call is expected to fail validation; no call here reaches a launch.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import long_context_verify_amd as L
from long_context_verify_amd import api

OK, INVALID, UNSUPPORTED, BAD_TREE, MISALIGNED, WORKSPACE = 0, 1, 2, 3, 4, 5
P = ctypes.c_void_p(0x10000)          # aligned fake device pointer (never dereferenced)
P_ODD = ctypes.c_void_p(0x10004)      # 4-byte aligned only
NULL = None


def test_library_file_exists_and_loads():
    assert os.path.exists(api.LIB_PATH), "run __graft_entry__.build() first"
    assert L.lib() is not None


def test_every_declared_function_is_exported():
    names = api.declared_functions()
    assert {"spec_verify_attention", "spec_window_attention", "spec_sample"} <= set(names)
    handle = ctypes.CDLL(api.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert set(names) == set(api._SIGNATURES)


def test_status_strings():
    assert L.status_str(0) == "SPEC_OK"
    assert L.status_str(4) == "SPEC_ERR_MISALIGNED"
    assert L.status_str(99) == "SPEC_ERR_UNKNOWN"


def _verify(q=P, k=P, v=P, out=P, lse=NULL, kv_len=NULL, parent=NULL, pstride=0, B=2, Hq=8,
            Hkv=2, n_q=5, D=128, L_cap=1000, dtype=1, scale=0.0, splits=0, ws=P, ws_bytes=0,
            err=NULL):
    return L.lib().spec_verify_attention(q, k, v, out, lse, kv_len, parent, pstride, B, Hq, Hkv,
                                         n_q, D, L_cap, dtype, scale, splits, ws, ws_bytes, err,
                                         NULL)


def test_verify_attention_argument_checks():
    assert _verify(B=0) == OK                      # empty batch: nothing to do
    assert _verify(Hq=7) == INVALID                # Hq % Hkv != 0
    assert _verify(D=96) == UNSUPPORTED
    assert _verify(n_q=65) == UNSUPPORTED
    assert _verify(n_q=0) == INVALID
    assert _verify(L_cap=4) == INVALID             # L_cap < n_q
    assert _verify(dtype=5) == INVALID
    assert _verify(splits=-1) == INVALID
    assert _verify(parent=P, pstride=3) == INVALID
    assert _verify(q=P_ODD) == MISALIGNED
    assert _verify(k=NULL) == MISALIGNED
    assert _verify(ws_bytes=16) == WORKSPACE       # far below the planned workspace
    assert _verify(ws=P_ODD, ws_bytes=1 << 40) == WORKSPACE
    # more than 2^22 work-groups: refused before the workspace is looked at
    assert _verify(B=4096, Hq=64, Hkv=64, L_cap=1 << 20, splits=65536) == UNSUPPORTED


def test_workspace_queries():
    import torch
    bf16 = torch.bfloat16
    a = L.verify_attention_workspace_bytes(8, 32, 8, 5, 128, 32768, bf16)
    b = L.verify_attention_workspace_bytes(8, 32, 8, 5, 128, 32768, bf16, num_splits=1)
    assert a > b > 0 and a % 256 == 0
    assert L.verify_attention_workspace_bytes(8, 32, 8, 5, 96, 32768, bf16) == 0
    assert L.verify_attention_auto_splits(8, 32, 8, 5, 128, 32768, bf16) >= 1
    assert L.window_attention_workspace_bytes(8, 32, 8, 128, 512, 4, bf16) > 0
    assert L.sample_workspace_bytes(8, 5, 128256) > 0
    assert L.sample_workspace_bytes(8, 0, 128256) == 0
    # More than 2^22 work-groups: refused (a zero size here, UNSUPPORTED at the call).
    assert L.verify_attention_workspace_bytes(4096, 64, 64, 5, 128, 1 << 20, bf16,
                                              num_splits=65536) == 0
    assert L.window_attention_workspace_bytes(8192, 64, 64, 128, 512, 4, bf16,
                                              num_splits=65536) == 0


def _paged(B=2, P_size=64, stride=16, num_pages=40, bt=P, kv_len=P, L_max=1000, ws_bytes=0):
    return L.lib().spec_verify_attention_paged(P, P, P, bt, stride, num_pages, P_size, P, NULL,
                                               kv_len, NULL, 0, B, 8, 2, 5, 128, L_max, 1, 0.0, 0,
                                               P, ws_bytes, NULL, NULL)


def test_verify_paged_argument_checks():
    assert _paged(B=0) == OK
    assert _paged(P_size=32) == UNSUPPORTED
    assert _paged(P_size=96) == UNSUPPORTED
    assert _paged(P_size=0) == INVALID
    assert _paged(stride=15) == INVALID          # ceil(1000 / 64) = 16 entries needed
    assert _paged(num_pages=0) == INVALID
    assert _paged(bt=NULL) == MISALIGNED
    assert _paged(kv_len=NULL) == MISALIGNED
    assert _paged() == WORKSPACE
    assert L.verify_attention_paged_workspace_bytes(2, 8, 2, 5, 128, 1000, 64, torch.bfloat16) > 0
    assert L.verify_attention_paged_workspace_bytes(2, 8, 2, 5, 128, 1000, 48, torch.bfloat16) == 0


def _window(B=2, Hq=8, Hkv=2, D=128, W=64, S=4, k_new=NULL, v_new=NULL, k_sink=P, ws_bytes=0,
            total_len=P, dtype=1):
    return L.lib().spec_window_attention(P, P, P, k_sink, P, k_new, v_new, total_len, P, NULL, B,
                                         Hq, Hkv, D, W, S, dtype, 0.0, 0, P, ws_bytes, NULL, NULL)


def test_window_attention_argument_checks():
    assert _window(B=0) == OK
    assert _window(W=0) == INVALID
    assert _window(S=-1) == INVALID
    assert _window(D=32) == UNSUPPORTED
    assert _window(k_new=P) == INVALID             # k_new without v_new
    assert _window(k_sink=NULL) == MISALIGNED      # sinks needed when S > 0
    assert _window(total_len=NULL) == MISALIGNED
    assert _window() == WORKSPACE


def _sample(B=2, N=5, V=1000, offset=0, parent=NULL, pstride=0, tgt=P, ws_bytes=0):
    return L.lib().spec_sample(tgt, P, P, parent, pstride, B, N, V, 1, offset, P, P, NULL, NULL, P,
                               ws_bytes, NULL, NULL)


def test_sample_argument_checks():
    assert _sample(B=0) == OK
    assert _sample(N=0) == INVALID
    assert _sample(N=257) == UNSUPPORTED
    assert _sample(V=0) == INVALID
    assert _sample(offset=1 << 30) == INVALID
    assert _sample(parent=P, pstride=4) == INVALID
    assert _sample(tgt=P_ODD) == MISALIGNED
    assert _sample() == WORKSPACE
    assert L.lib().spec_sample_bf16(P, P, P, NULL, 0, 2, 5, 1000, 1, 0, P, P, NULL, NULL, P, 0,
                                    NULL, NULL) == WORKSPACE
    for dt, rule, want in [(0, 1, WORKSPACE), (1, 0, WORKSPACE), (2, 0, INVALID), (0, 2, INVALID)]:
        assert L.lib().spec_sample_ex(P, P, dt, rule, P, NULL, 0, 2, 5, 1000, 1, 0, P, P, NULL,
                                      NULL, P, 0, NULL, NULL) == want
    assert L.lib().spec_sample_bf16(P_ODD, P, P, NULL, 0, 2, 5, 1000, 1, 0, P, P, NULL, NULL, P,
                                    0, NULL, NULL) == MISALIGNED


def _draft(B=2, V=1000, stride=0, node=1, offset=0, logits=P, tok=P, tstride=0, ws_bytes=0,
           dtype=0):
    return L.lib().spec_draft_sample(logits, dtype, stride, B, V, 1, offset, node, tok, tstride,
                                     NULL, P, ws_bytes, NULL, NULL)


def test_draft_sample_argument_checks():
    assert _draft(B=0) == OK
    assert _draft(V=0) == INVALID
    assert _draft(V=(1 << 27) + 1) == UNSUPPORTED
    assert _draft(node=-1) == INVALID
    assert _draft(offset=1 << 30) == INVALID
    assert _draft(stride=999) == INVALID
    assert _draft(tstride=-1) == INVALID
    assert _draft(logits=NULL) == MISALIGNED
    assert _draft(dtype=3) == INVALID
    assert _draft(logits=ctypes.c_void_p(0x10002)) == MISALIGNED
    assert _draft(logits=ctypes.c_void_p(0x10002), dtype=1) == WORKSPACE
    assert _draft(tok=ctypes.c_void_p(0x10002)) == MISALIGNED
    assert _draft() == WORKSPACE
    assert L.draft_sample_workspace_bytes(8, 128256) >= 8 * 16 * 20
    assert L.draft_sample_workspace_bytes(0, 10) == 0


def _commit(B=2, Hkv=2, n_q=5, D=128, L_cap=64, dtype=1, k=P, kv_len=P, path=NULL, count=P,
            total=NULL, appended=0):
    return L.lib().spec_kv_commit(k, P, kv_len, path, count, B, Hkv, n_q, D, L_cap, dtype, total,
                                  appended, NULL, NULL)


def test_kv_commit_argument_checks():
    assert _commit(B=0) == OK
    assert _commit(B=0, n_q=0) == INVALID
    assert _commit(n_q=65) == UNSUPPORTED
    assert _commit(D=96) == UNSUPPORTED
    assert _commit(L_cap=4) == INVALID
    assert _commit(dtype=7) == INVALID
    assert _commit(total=P, appended=6) == INVALID
    assert _commit(total=P, appended=-1) == INVALID
    assert _commit(k=P_ODD) == MISALIGNED
    assert _commit(kv_len=NULL) == MISALIGNED
    assert _commit(count=NULL) == MISALIGNED


@pytest.mark.parametrize("parent,single,expect", [
    ([-1, 0, 0, 1, 3], True, OK),
    ([-1, 0, 2], True, BAD_TREE),          # parent not before child
    ([-1, -1, 0], True, BAD_TREE),         # second root
    ([-1, -1, 0], False, OK),              # forests are fine for attention
    ([0, 0], False, BAD_TREE),             # node 0 cannot have a parent
    ([-1, -2], False, BAD_TREE),
])
def test_validate_tree(parent, single, expect):
    assert L.validate_tree(np.array(parent), single) == expect


def test_validate_tree_null():
    assert L.lib().spec_validate_tree(NULL, 3, 1) == INVALID


def test_binding_refuses_host_tensors():
    """No CPU fallback: every entry point refuses tensors that are not on a
    HIP device before any library call."""
    q = torch.zeros(1, 4, 5, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        L.verify_attention(q, k, k)
    with pytest.raises(ValueError, match="HIP device"):
        L.window_attention(q[:, :, :1], k, k, k[:, :, :4], k[:, :, :4], [10])
    logits = torch.zeros(2, 5, 100)
    with pytest.raises(ValueError, match="HIP device"):
        L.spec_sample(logits, logits, torch.zeros(2, 5, dtype=torch.int32))
    with pytest.raises(ValueError, match="HIP device"):
        L.draft_sample(logits[:, 0], node=1)
    with pytest.raises(ValueError, match="HIP device"):
        L.kv_commit(k, k, torch.zeros(1, dtype=torch.int32), torch.ones(1, dtype=torch.int32), 5)


def test_bench_refuses_more_than_one_gpu():
    """The measured path is one GPU's: --gpus N > 1 exits with a message and
    touches no device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def _i32(*shape):
    return torch.zeros(*shape, dtype=torch.int32)


# Each case: a call whose tensors disagree with the sizes the call derives
# from its primary inputs.  The binding must refuse it (ValueError naming the
# argument) before the device check and before any library call, since the
# C ABI sees only raw pointers.
_Q, _K = _bf(2, 8, 5, 64), _bf(2, 2, 100, 64)
_WQ, _RING, _SINK = _bf(2, 8, 1, 64), _bf(2, 2, 16, 64), _bf(2, 2, 4, 64)
_LOG, _TOK = torch.zeros(2, 5, 100), _i32(2, 5)
SHAPE_CASES = [
    ("verify v_cache", lambda: L.verify_attention(_Q, _K, _bf(2, 2, 99, 64)), "v_cache"),
    ("verify k batch", lambda: L.verify_attention(_Q, _bf(3, 2, 100, 64), _bf(3, 2, 100, 64)),
     "k_cache"),
    ("verify k head dim", lambda: L.verify_attention(_Q, _bf(2, 2, 100, 128),
                                                     _bf(2, 2, 100, 128)), "k_cache"),
    ("verify dtype", lambda: L.verify_attention(_Q, _K.float(), _K.float()), "dtype"),
    ("verify kv_len", lambda: L.verify_attention(_Q, _K, _K, kv_len=_i32(3)), "kv_len"),
    ("verify kv_len list", lambda: L.verify_attention(_Q, _K, _K, kv_len=[5, 5, 5]), "kv_len"),
    ("verify out", lambda: L.verify_attention(_Q, _K, _K, out=_bf(2, 8, 5, 32)), "out"),
    ("verify out dtype", lambda: L.verify_attention(_Q, _K, _K, out=_Q.float()), "out"),
    ("verify lse", lambda: L.verify_attention(_Q, _K, _K, lse=torch.zeros(2, 8, 4)), "lse"),
    ("verify dev_err", lambda: L.verify_attention(_Q, _K, _K,
                                                  dev_err=torch.zeros(1, dtype=torch.int64)),
     "dev_err"),
    ("verify dev_err empty", lambda: L.verify_attention(_Q, _K, _K, dev_err=_i32(0)), "dev_err"),
    ("verify parent", lambda: L.verify_attention(_Q, _K, _K, parent=[-1, 0, 1]), "parent"),
    ("paged v_pages", lambda: L.verify_attention_paged(_Q, _bf(9, 2, 64, 64), _bf(9, 2, 64, 32),
                                                       _i32(2, 2), _i32(2), 100), "v_pages"),
    ("paged kv_len", lambda: L.verify_attention_paged(_Q, _bf(9, 2, 64, 64), _bf(9, 2, 64, 64),
                                                      _i32(2, 2), _i32(4), 100), "kv_len"),
    ("paged table rows", lambda: L.verify_attention_paged(_Q, _bf(9, 2, 64, 64),
                                                          _bf(9, 2, 64, 64), _i32(3, 2),
                                                          _i32(2), 100), "block_table"),
    ("paged table dtype", lambda: L.verify_attention_paged(
        _Q, _bf(9, 2, 64, 64), _bf(9, 2, 64, 64), torch.zeros(2, 2, dtype=torch.int64), _i32(2),
        100), "block_table"),
    ("window q rows", lambda: L.window_attention(_bf(2, 8, 2, 64), _RING, _RING, _SINK, _SINK,
                                                 [20, 20]), "q"),
    ("window ring dtype", lambda: L.window_attention(_WQ.float(), _RING, _RING, _SINK, _SINK,
                                                     [20, 20]), "k_ring"),
    ("window v_ring", lambda: L.window_attention(_WQ, _RING, _bf(2, 2, 8, 64), _SINK, _SINK,
                                                 [20, 20]), "v_ring"),
    ("window sink", lambda: L.window_attention(_WQ, _RING, _RING, _SINK, _bf(2, 2, 3, 64),
                                               [20, 20]), "v_sink"),
    ("window sink pair", lambda: L.window_attention(_WQ, _RING, _RING, _SINK, None, [20, 20]),
     "v_sink"),
    ("window new", lambda: L.window_attention(_WQ, _RING, _RING, _SINK, _SINK, [20, 20],
                                              k_new=_bf(2, 2, 2, 64), v_new=_bf(2, 2, 2, 64)),
     "k_new"),
    ("window new pair", lambda: L.window_attention(_WQ, _RING, _RING, _SINK, _SINK, [20, 20],
                                                   k_new=_bf(2, 2, 1, 64)), "v_new"),
    ("window total_len", lambda: L.window_attention(_WQ, _RING, _RING, _SINK, _SINK, _i32(3)),
     "total_len"),
    ("window out", lambda: L.window_attention(_WQ, _RING, _RING, _SINK, _SINK, [20, 20],
                                              out=_bf(2, 8, 1, 32)), "out"),
    ("window lse", lambda: L.window_attention(_WQ, _RING, _RING, _SINK, _SINK, [20, 20],
                                              lse=torch.zeros(2, 8)), "lse"),
    ("sample draft", lambda: L.spec_sample(_LOG, torch.zeros(2, 5, 99), _TOK), "draft_logits"),
    ("sample tokens", lambda: L.spec_sample(_LOG, _LOG, _i32(2, 4)), "tokens"),
    ("sample tokens dtype", lambda: L.spec_sample(_LOG, _LOG, _TOK.long()), "tokens"),
    ("sample out_tokens", lambda: L.spec_sample(_LOG, _LOG, _TOK, out_tokens=_i32(2, 6)),
     "out_tokens"),
    ("sample out_count", lambda: L.spec_sample(_LOG, _LOG, _TOK, out_count=_i32(1)),
     "out_count"),
    ("sample out_path", lambda: L.spec_sample(_LOG, _LOG, _TOK, out_path=_i32(5, 2)),
     "out_path"),
    ("sample out_accept", lambda: L.spec_sample(_LOG, _LOG, _TOK, out_accept=_i32(2, 5)),
     "out_accept"),
    ("sample dev_err", lambda: L.spec_sample(_LOG, _LOG, _TOK, dev_err=torch.zeros(1)),
     "dev_err"),
    ("sample parent", lambda: L.spec_sample(_LOG, _LOG, _TOK, parent=[-1, 0, 0]), "parent"),
    ("draft out_token", lambda: L.draft_sample(_LOG[:, 0], 1, out_token=_i32(3)), "out_token"),
    ("draft out_logprob", lambda: L.draft_sample(_LOG[:, 0], 1, out_logprob=torch.zeros(3)),
     "out_logprob"),
    ("commit v", lambda: L.kv_commit(_K, _bf(2, 2, 100, 32), _i32(2), _i32(2), 5), "v_cache"),
    ("commit kv_len", lambda: L.kv_commit(_K, _K, _i32(3), _i32(2), 5), "kv_len"),
    ("commit count", lambda: L.kv_commit(_K, _K, _i32(2), _i32(1), 5), "count"),
    ("commit path", lambda: L.kv_commit(_K, _K, _i32(2), _i32(2), 5, path=_i32(2, 4)), "path"),
    ("commit total", lambda: L.kv_commit(_K, _K, _i32(2), _i32(2), 5,
                                         draft_total_len=_i32(2, 1)), "draft_total_len"),
]


@pytest.mark.parametrize("case", SHAPE_CASES, ids=[c[0] for c in SHAPE_CASES])
def test_binding_refuses_mismatched_shapes(case):
    _, call, word = case
    with pytest.raises(ValueError) as e:
        call()
    msg = str(e.value)
    assert "HIP device" not in msg, f"shape mismatch not caught before the device check: {msg}"
    assert word.split("_")[0] in msg or word in msg, msg


def test_sample_noalloc_argument_checks():
    """Host checks of the no-allocation sampling call: sizes whose workspace
    exceeds the library's scratch array are refused before any HIP call."""
    def call(B=2, N=5, V=1000, dt=0, rule=0, tgt=P, offset=0):
        return L.lib().spec_sample_noalloc(tgt, P, dt, rule, P, NULL, 0, B, N, V, 1, offset, P,
                                           P, NULL, NULL, NULL, NULL)
    assert call(B=0) == OK
    assert call(N=0) == INVALID
    assert call(dt=2) == INVALID
    assert call(rule=2) == INVALID
    assert call(offset=1 << 30) == INVALID
    assert call(tgt=P_ODD) == MISALIGNED
    assert L.sample_workspace_bytes(4096, 2, 1000) > 4 << 20
    assert call(B=4096, N=2, V=1000) == UNSUPPORTED
    assert call(B=64, N=8, V=1 << 27) == UNSUPPORTED
