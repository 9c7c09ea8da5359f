"""Helpers shared by the GPU parity tests (no test functions here)."""

import sys

import numpy as np
import torch

from oracle.attention import verify_attention as oracle_verify


def say(msg):
    """Print and flush the case name before each GPU step."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def cpu64(t):
    return t.detach().to("cpu").double().numpy()


def tol_for(dtype):
    """Max-abs tolerances: fp32 1e-5 (outputs and lse); bf16 2e-2 on outputs, 1e-2 on lse."""
    return (1e-5, 1e-5) if dtype == torch.float32 else (2e-2, 1e-2)


def assert_attention_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    ta, tl = tol_for(dtype)
    og = cpu64(o_gpu)
    err = np.max(np.abs(og - o_ref))
    assert err <= ta, f"{what}: max abs out error {err:.3e} > {ta}"
    if dtype == torch.bfloat16:
        rel = np.linalg.norm(og - o_ref) / max(np.linalg.norm(o_ref), 1e-30)
        assert rel <= 1e-2, f"{what}: relative Frobenius error {rel:.3e} > 1e-2"
    if lse_gpu is not None:
        le = np.max(np.abs(cpu64(lse_gpu) - lse_ref))
        assert le <= tl, f"{what}: max abs lse error {le:.3e} > {tl}"
    return err


def oracle_unit(q, k, v, kv_len, parent, b, hk, g):
    """Oracle outputs of one (sequence, kv head) unit: rows of heads hk*g .. hk*g+g-1."""
    qs = q[b:b + 1, hk * g:(hk + 1) * g].cpu()
    ks = k[b:b + 1, hk:hk + 1].cpu()
    vs = v[b:b + 1, hk:hk + 1].cpu()
    kl = None if kv_len is None else [int(kv_len[b])]
    par = None
    if parent is not None:
        par = np.asarray(parent.cpu() if hasattr(parent, "cpu") else parent)
        if par.ndim == 2:
            par = par[b]
    return oracle_verify(qs, ks, vs, kl, par)
