"""ctypes binding of ``libspecverify.so`` -- argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
checks tensor dtypes and contiguity, allocates outputs and workspaces with
torch (device memory is the only thing torch provides), and passes raw
pointers plus torch's current HIP stream to the C entry points declared in
``include/spec_verify.h``.  There is no fallback: if the library is missing
or the tensors are not on a HIP device, the call raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIB selects another build of the same library (the sanitized one).
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(HERE, "libspecverify.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "spec_verify.h")

SPEC_F32, SPEC_BF16 = 0, 1
_DTYPES = {torch.float32: SPEC_F32, torch.bfloat16: SPEC_BF16}

_vp, _i32, _u64, _f32, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64,
                              ctypes.c_float, ctypes.c_size_t)

_SIGNATURES = {
    "spec_verify_attention": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                     _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp, _vp]),
    "spec_verify_attention_workspace": (_sz, [_i32] * 8),
    "spec_verify_attention_auto_splits": (_i32, [_i32] * 7),
    "spec_verify_attention_paged": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                           _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                           _i32, _vp, _sz, _vp, _vp]),
    "spec_verify_attention_paged_workspace": (_sz, [_i32] * 9),
    "spec_window_attention": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                     _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp, _vp]),
    "spec_window_attention_workspace": (_sz, [_i32] * 8),
    "spec_sample": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _u64, _u64, _vp, _vp, _vp,
                           _vp, _vp, _sz, _vp, _vp]),
    "spec_sample_workspace": (_sz, [_i32] * 3),
    "spec_sample_ex": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _u64, _u64,
                              _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "spec_sample_noalloc": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _u64,
                                   _u64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "spec_sample_bf16": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _u64, _u64, _vp, _vp,
                                _vp, _vp, _vp, _sz, _vp, _vp]),
    "spec_draft_sample": (_i32, [_vp, _i32, ctypes.c_int64, _i32, _i32, _u64, _u64, _i32, _vp,
                                 _i32, _vp, _vp, _sz, _vp, _vp]),
    "spec_draft_sample_workspace": (_sz, [_i32, _i32]),
    "spec_kv_commit": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp,
                              _i32, _vp, _vp]),
    "spec_validate_tree": (_i32, [_vp, _i32, _i32]),
    "spec_status_str": (ctypes.c_char_p, [_i32]),
}

_lib = None


class SpecError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


def declared_functions() -> list:
    """Names of the functions declared in include/spec_verify.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(spec_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def lib():
    """Load the built library once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_verify_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().spec_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise SpecError(status, where)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_gpu(*ts, strided_ok=()):
    for i, t in enumerate(ts):
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on a HIP device")
        if t is not None and i not in strided_ok and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    """A caller's workspace (zero-filled before its first use, then reusable
    by any later call on the same stream), or a fresh zero-filled one."""
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on a HIP device")
        if _nbytes(workspace) < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _expect(t, name: str, shape=None, dtype=None, min_numel: int = 0):
    """Shape and dtype check of one tensor argument (None passes).  The C ABI
    sees raw pointers only, so every size the kernels will index with is
    checked here against the sizes derived from the call's primary inputs."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} needs at least {min_numel} elements")


def _expect_dev_err(dev_err):
    _expect(dev_err, "dev_err", dtype=torch.int32, min_numel=1)


def _expect_dims(t, name: str, ndim: int):
    if not isinstance(t, torch.Tensor) or t.dim() != ndim:
        raise ValueError(f"{name} must be a {ndim}-d tensor")


def _check_parent(parent, B, n):
    """A parent array is [n] (shared) or [B, n] (per sequence)."""
    if parent is None:
        return
    shape = tuple(parent.shape) if hasattr(parent, "shape") else tuple(np.shape(parent))
    if shape != (n,) and shape != (B, n):
        raise ValueError(f"parent has shape {shape}, expected ({n},) or ({B}, {n})")


def _parent_arg(parent, B, n, device):
    if parent is None:
        return None, 0
    _check_parent(parent, B, n)
    pt = torch.as_tensor(parent, dtype=torch.int32, device=device).contiguous()
    return (pt, 0) if pt.dim() == 1 else (pt, n)


def verify_attention_workspace_bytes(B, Hq, Hkv, n_q, D, L_cap, dtype, num_splits=0) -> int:
    return int(lib().spec_verify_attention_workspace(B, Hq, Hkv, n_q, D, L_cap, _DTYPES[dtype],
                                                     num_splits))


def verify_attention_auto_splits(B, Hq, Hkv, n_q, D, L_cap, dtype) -> int:
    return int(lib().spec_verify_attention_auto_splits(B, Hq, Hkv, n_q, D, L_cap, _DTYPES[dtype]))


def verify_attention(q, k_cache, v_cache, kv_len=None, parent=None, scale: float = 0.0,
                     num_splits: int = 0, out=None, lse=None, workspace=None, dev_err=None,
                     want_lse: bool = True):
    """spec_verify_attention on torch tensors.  Returns (out, lse or None)."""
    _expect_dims(q, "q", 4)
    _expect_dims(k_cache, "k_cache", 4)
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, Hq, n_q, D = q.shape
    Hkv, L_cap = k_cache.shape[1], k_cache.shape[2]
    _expect(k_cache, "k_cache", (B, Hkv, L_cap, D))
    _expect(v_cache, "v_cache", (B, Hkv, L_cap, D))
    if isinstance(kv_len, torch.Tensor):
        _expect(kv_len, "kv_len", (B,))
    elif kv_len is not None and len(kv_len) != B:
        raise ValueError("kv_len must have B entries")
    _expect(out, "out", q.shape, q.dtype)
    _expect(lse, "lse", (B, Hq, n_q), torch.float32)
    _expect_dev_err(dev_err)
    _check_parent(parent, B, n_q)
    _need_gpu(q, k_cache, v_cache, kv_len if isinstance(kv_len, torch.Tensor) else None, out, lse,
              dev_err)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, n_q, dtype=torch.float32, device=dev)
    if kv_len is not None:
        kv_len = torch.as_tensor(kv_len, dtype=torch.int32, device=dev).contiguous()
    par, pstride = _parent_arg(parent, B, n_q, dev)
    nbytes = verify_attention_workspace_bytes(B, Hq, Hkv, n_q, D, L_cap, q.dtype, num_splits)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().spec_verify_attention(
        _p(q), _p(k_cache), _p(v_cache), _p(out), _p(lse), _p(kv_len), _p(par), pstride,
        B, Hq, Hkv, n_q, D, L_cap, _DTYPES[q.dtype], float(scale), int(num_splits), _p(ws),
        _nbytes(ws), _p(dev_err), _stream(dev))
    _check(st, "spec_verify_attention")
    return out, lse


def verify_attention_paged_workspace_bytes(B, Hq, Hkv, n_q, D, L_max, page_size, dtype,
                                           num_splits=0) -> int:
    return int(lib().spec_verify_attention_paged_workspace(B, Hq, Hkv, n_q, D, L_max, page_size,
                                                           _DTYPES[dtype], num_splits))


def verify_attention_paged(q, k_pages, v_pages, block_table, kv_len, L_max: int, parent=None,
                           scale: float = 0.0, num_splits: int = 0, out=None, lse=None,
                           workspace=None, dev_err=None, want_lse: bool = True):
    """spec_verify_attention_paged on torch tensors.

    k_pages, v_pages: [num_pages, Hkv, P, D]; block_table: [B, stride] int32;
    kv_len: [B] int32 (required).  Returns (out, lse or None)."""
    _expect_dims(q, "q", 4)
    _expect_dims(k_pages, "k_pages", 4)
    _expect_dims(block_table, "block_table", 2)
    if q.dtype not in _DTYPES or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, Hq, n_q, D = q.shape
    num_pages, Hkv, P = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _expect(k_pages, "k_pages", (num_pages, Hkv, P, D))
    _expect(v_pages, "v_pages", (num_pages, Hkv, P, D))
    _expect(block_table, "block_table", (B, block_table.shape[1]), torch.int32)
    _expect(kv_len, "kv_len", (B,), torch.int32)
    _expect(out, "out", q.shape, q.dtype)
    _expect(lse, "lse", (B, Hq, n_q), torch.float32)
    _expect_dev_err(dev_err)
    _check_parent(parent, B, n_q)
    _need_gpu(q, k_pages, v_pages, block_table, kv_len, out, lse, dev_err)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, n_q, dtype=torch.float32, device=dev)
    par, pstride = _parent_arg(parent, B, n_q, dev)
    nbytes = verify_attention_paged_workspace_bytes(B, Hq, Hkv, n_q, D, L_max, P, q.dtype,
                                                    num_splits)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().spec_verify_attention_paged(
        _p(q), _p(k_pages), _p(v_pages), _p(block_table), int(block_table.shape[1]), num_pages, P,
        _p(out), _p(lse), _p(kv_len), _p(par), pstride, B, Hq, Hkv, n_q, D, int(L_max),
        _DTYPES[q.dtype], float(scale), int(num_splits), _p(ws), _nbytes(ws), _p(dev_err),
        _stream(dev))
    _check(st, "spec_verify_attention_paged")
    return out, lse


def window_attention_workspace_bytes(B, Hq, Hkv, D, W, S, dtype, num_splits=0) -> int:
    return int(lib().spec_window_attention_workspace(B, Hq, Hkv, D, W, S, _DTYPES[dtype],
                                                     num_splits))


def window_attention(q, k_ring, v_ring, k_sink, v_sink, total_len, k_new=None, v_new=None,
                     scale: float = 0.0, num_splits: int = 0, out=None, lse=None,
                     workspace=None, dev_err=None, want_lse: bool = True):
    """spec_window_attention on torch tensors.  Returns (out, lse or None)."""
    _expect_dims(q, "q", 4)
    _expect_dims(k_ring, "k_ring", 4)
    if q.dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    B, Hq, _, D = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    _expect(q, "q", (B, Hq, 1, D))
    _expect(k_ring, "k_ring", (B, Hkv, W, D), q.dtype)
    _expect(v_ring, "v_ring", (B, Hkv, W, D), q.dtype)
    if (k_sink is None) != (v_sink is None):
        raise ValueError("k_sink and v_sink must both be given or both be None")
    if k_sink is not None:
        _expect_dims(k_sink, "k_sink", 4)
    S = 0 if k_sink is None else k_sink.shape[2]
    _expect(k_sink, "k_sink", (B, Hkv, S, D), q.dtype)
    _expect(v_sink, "v_sink", (B, Hkv, S, D), q.dtype)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    _expect(k_new, "k_new", (B, Hkv, 1, D), q.dtype)
    _expect(v_new, "v_new", (B, Hkv, 1, D), q.dtype)
    if isinstance(total_len, torch.Tensor):
        _expect(total_len, "total_len", (B,))
    elif len(total_len) != B:
        raise ValueError("total_len must have B entries")
    _expect(out, "out", q.shape, q.dtype)
    _expect(lse, "lse", (B, Hq, 1), torch.float32)
    _expect_dev_err(dev_err)
    _need_gpu(q, k_ring, v_ring, k_sink, v_sink, k_new, v_new,
              total_len if isinstance(total_len, torch.Tensor) else None, out, lse, dev_err)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, 1, dtype=torch.float32, device=dev)
    tl = torch.as_tensor(total_len, dtype=torch.int32, device=dev).contiguous()
    nbytes = window_attention_workspace_bytes(B, Hq, Hkv, D, W, S, q.dtype, num_splits)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().spec_window_attention(
        _p(q), _p(k_ring), _p(v_ring), _p(k_sink), _p(v_sink), _p(k_new), _p(v_new), _p(tl),
        _p(out), _p(lse), B, Hq, Hkv, D, W, S, _DTYPES[q.dtype], float(scale), int(num_splits),
        _p(ws), _nbytes(ws), _p(dev_err), _stream(dev))
    _check(st, "spec_window_attention")
    return out, lse


def sample_workspace_bytes(B, N, V) -> int:
    return int(lib().spec_sample_workspace(B, N, V))


def spec_sample(target_logits, draft_logits, tokens, parent=None, seed: int = 0, offset: int = 0,
                out_tokens=None, out_count=None, out_path=None, out_accept=None,
                workspace=None, dev_err=None, want_path: bool = True, want_accept: bool = True,
                siblings: str = "first"):
    """spec_sample on torch tensors.  Returns dict(out_tokens, out_count, out_path, out_accept).

    fp32 logits go to spec_sample, bf16 to spec_sample_bf16; siblings="lossless"
    selects spec_sample_ex's lossless sibling rule."""
    if siblings not in ("first", "lossless"):
        raise ValueError("siblings must be 'first' or 'lossless'")
    _expect_dims(target_logits, "target_logits", 3)
    if target_logits.dtype not in _DTYPES or draft_logits.dtype != target_logits.dtype:
        raise ValueError("logits must be float32 or bfloat16 (both the same)")
    B, N, V = target_logits.shape
    _expect(draft_logits, "draft_logits", (B, N, V))
    _expect(tokens, "tokens", (B, N), torch.int32)
    _expect(out_tokens, "out_tokens", (B, N), torch.int32)
    _expect(out_count, "out_count", (B,), torch.int32)
    _expect(out_path, "out_path", (B, N), torch.int32)
    _expect(out_accept, "out_accept", (B, N), torch.uint8)
    _expect_dev_err(dev_err)
    _check_parent(parent, B, N)
    _need_gpu(target_logits, draft_logits, tokens, out_tokens, out_count, out_path, out_accept,
              dev_err)
    dev = target_logits.device
    if out_tokens is None:
        out_tokens = torch.empty(B, N, dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty(B, dtype=torch.int32, device=dev)
    if out_path is None and want_path:
        out_path = torch.empty(B, N, dtype=torch.int32, device=dev)
    if out_accept is None and want_accept:
        out_accept = torch.empty(B, N, dtype=torch.uint8, device=dev)
    par, pstride = _parent_arg(parent, B, N, dev)
    ws = _workspace(sample_workspace_bytes(B, N, V), dev, workspace)
    args = (_p(tokens), _p(par), pstride, B, N, V, int(seed) & (2**64 - 1), int(offset),
            _p(out_tokens), _p(out_count), _p(out_path), _p(out_accept), _p(ws), _nbytes(ws),
            _p(dev_err), _stream(dev))
    if siblings == "lossless":
        st = lib().spec_sample_ex(_p(target_logits), _p(draft_logits),
                                  _DTYPES[target_logits.dtype], 1, *args)
    elif target_logits.dtype == torch.bfloat16:
        st = lib().spec_sample_bf16(_p(target_logits), _p(draft_logits), *args)
    else:
        st = lib().spec_sample(_p(target_logits), _p(draft_logits), *args)
    _check(st, "spec_sample")
    return {"out_tokens": out_tokens, "out_count": out_count, "out_path": out_path,
            "out_accept": out_accept}


def spec_sample_noalloc(target_logits, draft_logits, tokens, parent=None, seed: int = 0,
                        offset: int = 0, out_tokens=None, out_count=None, out_path=None,
                        out_accept=None, dev_err=None, want_path: bool = True,
                        want_accept: bool = True, siblings: str = "first"):
    """spec_sample_noalloc on torch tensors: spec_sample without a workspace (the
    library's own per-device scratch array is used; outputs are still the
    caller's).  Returns dict(out_tokens, out_count, out_path, out_accept)."""
    if siblings not in ("first", "lossless"):
        raise ValueError("siblings must be 'first' or 'lossless'")
    _expect_dims(target_logits, "target_logits", 3)
    if target_logits.dtype not in _DTYPES or draft_logits.dtype != target_logits.dtype:
        raise ValueError("logits must be float32 or bfloat16 (both the same)")
    B, N, V = target_logits.shape
    _expect(draft_logits, "draft_logits", (B, N, V))
    _expect(tokens, "tokens", (B, N), torch.int32)
    _expect(out_tokens, "out_tokens", (B, N), torch.int32)
    _expect(out_count, "out_count", (B,), torch.int32)
    _expect(out_path, "out_path", (B, N), torch.int32)
    _expect(out_accept, "out_accept", (B, N), torch.uint8)
    _expect_dev_err(dev_err)
    _check_parent(parent, B, N)
    _need_gpu(target_logits, draft_logits, tokens, out_tokens, out_count, out_path, out_accept,
              dev_err)
    dev = target_logits.device
    if out_tokens is None:
        out_tokens = torch.empty(B, N, dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty(B, dtype=torch.int32, device=dev)
    if out_path is None and want_path:
        out_path = torch.empty(B, N, dtype=torch.int32, device=dev)
    if out_accept is None and want_accept:
        out_accept = torch.empty(B, N, dtype=torch.uint8, device=dev)
    par, pstride = _parent_arg(parent, B, N, dev)
    st = lib().spec_sample_noalloc(
        _p(target_logits), _p(draft_logits), _DTYPES[target_logits.dtype],
        1 if siblings == "lossless" else 0, _p(tokens), _p(par), pstride, B, N, V,
        int(seed) & (2**64 - 1), int(offset), _p(out_tokens), _p(out_count), _p(out_path),
        _p(out_accept), _p(dev_err), _stream(dev))
    _check(st, "spec_sample_noalloc")
    return {"out_tokens": out_tokens, "out_count": out_count, "out_path": out_path,
            "out_accept": out_accept}


def draft_sample_workspace_bytes(B, V) -> int:
    return int(lib().spec_draft_sample_workspace(B, V))


def draft_sample(draft_logits, node: int, seed: int = 0, offset: int = 0, out_token=None,
                 out_logprob=None, workspace=None, dev_err=None, want_logprob: bool = True):
    """spec_draft_sample on torch tensors.

    ``draft_logits`` is [B, V] fp32 whose rows may be strided (e.g. ``x[:, u]``
    of a [B, N, V] tensor); ``out_token`` may be a strided column of a [B, N]
    int32 tensor.  Returns (out_token, out_logprob)."""
    if draft_logits.dtype not in _DTYPES or draft_logits.dim() != 2:
        raise ValueError("draft_logits must be a [B, V] float32 or bfloat16 tensor")
    if draft_logits.stride(1) != 1:
        raise ValueError("draft_logits rows must be contiguous")
    B, V = draft_logits.shape
    if out_token is not None and (out_token.dtype != torch.int32 or out_token.dim() != 1
                                  or out_token.numel() != B):
        raise ValueError("out_token must be [B] int32")
    _expect(out_logprob, "out_logprob", (B,), torch.float32)
    _expect_dev_err(dev_err)
    _need_gpu(draft_logits, out_token, out_logprob, dev_err, strided_ok=(0, 1))
    dev = draft_logits.device
    if out_token is None:
        out_token = torch.empty(B, dtype=torch.int32, device=dev)
    if B > 1 and (draft_logits.stride(0) < V or out_token.stride(0) < 1):
        raise ValueError("rows of draft_logits and entries of out_token must not overlap")
    if out_logprob is None and want_logprob:
        out_logprob = torch.empty(B, dtype=torch.float32, device=dev)
    ws = _workspace(draft_sample_workspace_bytes(B, V), dev, workspace)
    st = lib().spec_draft_sample(
        _p(draft_logits), _DTYPES[draft_logits.dtype], int(draft_logits.stride(0)) if B > 1 else V,
        B, V,
        int(seed) & (2**64 - 1), int(offset), int(node), _p(out_token),
        int(out_token.stride(0)) if B > 1 else 1, _p(out_logprob), _p(ws), _nbytes(ws),
        _p(dev_err), _stream(dev))
    _check(st, "spec_draft_sample")
    return out_token, out_logprob


def kv_commit(k_cache, v_cache, kv_len, count, n_q: int, path=None, draft_total_len=None,
              draft_appended: int = 0, dev_err=None):
    """spec_kv_commit on torch tensors; updates k_cache, v_cache, kv_len (and
    draft_total_len) in place.  ``path`` is [B, n_q] (spec_sample's out_path)
    or None for a chain."""
    _expect_dims(k_cache, "k_cache", 4)
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    if k_cache.dtype not in _DTYPES:
        raise ValueError("caches must be float32 or bfloat16")
    B, Hkv, L_cap, D = k_cache.shape
    if kv_len is None or count is None:
        raise ValueError("kv_len and count are required")
    _expect(kv_len, "kv_len", (B,), torch.int32)
    _expect(count, "count", (B,), torch.int32)
    _expect(path, "path", (B, n_q), torch.int32)
    _expect(draft_total_len, "draft_total_len", (B,), torch.int32)
    _expect_dev_err(dev_err)
    _need_gpu(k_cache, v_cache, kv_len, count, path, draft_total_len, dev_err)
    st = lib().spec_kv_commit(
        _p(k_cache), _p(v_cache), _p(kv_len), _p(path), _p(count), B, Hkv, int(n_q), D, L_cap,
        _DTYPES[k_cache.dtype], _p(draft_total_len), int(draft_appended), _p(dev_err),
        _stream(k_cache.device))
    _check(st, "spec_kv_commit")


def validate_tree(parent, require_single_root: bool = True) -> int:
    """spec_validate_tree on a host parent array; returns the status code."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    return int(lib().spec_validate_tree(arr.ctypes.data_as(ctypes.c_void_p), int(arr.size),
                                        int(bool(require_single_root))))
