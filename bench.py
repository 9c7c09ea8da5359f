#!/usr/bin/env python3
"""Benchmark of one speculative verification step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input.
The default workload is the largest one that fits one GPU, a 70B-class GQA
layer at high batch (batch 64, 64 query heads, 8 KV heads, head dim 128,
bf16, 16384-token context, gamma = 3; 4 GiB of K/V):

  1. spec_verify_attention  the gamma+1 = 4 block queries of every sequence
                            against its KV cache (causal chain);
  2. spec_window_attention  one draft-step query against 4 sink tokens and a
                            W-slot ring (only workloads that have a draft
                            window: the 8B/32K and 128K shapes);
  3. spec_sample            acceptance test + residual/bonus draw over a
                            128256-token vocabulary (4 target rows and 3 draft
                            rows per sequence at the default).

All inputs are resident in HBM before the timed region.  The printed value is
verified draft tokens per second (batch * gamma per step, host clock around K
back-to-back steps).  Each step's verify call streams more than the 256 MB
Infinity Cache (537 MB to 4 GiB of K/V), so every step meets its sampling
logits in HBM, not in the cache.

Per-op device times come from HIP events on the stream the library launches
on (torch's current stream), with all calls queued behind a GPU sleep so host
launch latency cannot leak in:

* ops whose inputs exceed 768 MB: K back-to-back calls between one pair of
  events;
* smaller ops: K calls back to back (``us_warm``: their inputs may sit in the
  Infinity Cache), and K calls each preceded by a 512 MB read of an unrelated
  buffer, minus K such reads alone (``us``: inputs from HBM).

Also reported: the fraction of a stream-copy rate measured in the same run,
the other workloads' verify and sampling figures (``workloads``), the draft
window's cost against the context length next to full-cache n_q = 1 attention
(``window_scaling``), and the fp64 oracle timed on a bounded sample of the
headline workload on the host cores (``cpu_baseline``).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--page-size P] [--logits f32|bf16] [--siblings first|lossless]
                       [--cpu-budget SECONDS] [--copy-probe-mib MIB]
                       [--no-others] [--no-window-scaling] [--window-scaling-only]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix rate, vendor figure
METRIC = "verify-attn KV GB/s (% HBM peak) + verified draft tokens/sec, 1 MI355X"
DEFAULT_WORKLOAD = "llama70b_16k_chain_b64"
BIG_OP_BYTES = 768 << 20    # inputs above this cannot stay in the 256 MB Infinity Cache


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["long_context_verify_amd/csrc/attention.hip",
                  "long_context_verify_amd/csrc/spec_common.hpp",
                  "long_context_verify_amd/csrc/spec_internal.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per launch of the verify kernel from the committed counter summary.

    The summary records the counter-derived bytes and the hash of the kernel
    sources they were taken with; if the sources changed since, the figure no
    longer describes this kernel and None is returned.
    """
    path = os.path.join(ROOT, "profiles", f"verify_attn_{workload}_hbm_counters.txt")
    try:
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("workload") != workload or fields.get("source_sha256") != kernel_source_sha256():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--cpu-budget", type=float, default=12.0,
                   help="seconds of oracle work for the CPU baseline (0 disables it)")
    p.add_argument("--page-size", type=int, default=0,
                   help="read the verify cache through a block table of pages of this many "
                        "keys (a seeded shuffle of the contiguous cache); 0 = contiguous")
    p.add_argument("--siblings", choices=["first", "lossless"], default="first",
                   help="sibling rule of the sampling tail on candidate trees")
    p.add_argument("--logits", choices=["f32", "bf16"], default="f32",
                   help="dtype of the target and draft logits given to the sampling calls")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run plain device copies of this many MiB (calibrates HBM "
                        "byte counters: the copy reads and writes exactly this much)")
    p.add_argument("--no-others", action="store_true",
                   help="skip the verify and sampling figures of the other workloads")
    p.add_argument("--no-window-scaling", action="store_true",
                   help="skip the window-vs-context scaling run")
    p.add_argument("--window-scaling-only", action="store_true",
                   help="run only the window-vs-context scaling run and print its JSON")
    return p.parse_args()


# ---------------------------------------------------------------------------
# Device timing
# ---------------------------------------------------------------------------
class Timer:
    """Mean device time per call, from HIP events on the library's stream."""

    def __init__(self, dev):
        import torch
        self.torch = torch
        self.stream = torch.cuda.current_stream(dev)
        # 512 MB of unrelated data: reading it evicts the 256 MB Infinity Cache.
        self.flush_buf = torch.ones(128 << 20, dtype=torch.float32, device=dev)

    def flush(self):
        self.flush_buf.amax()

    def _bracket(self, body, n, warm=3):
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.05))   # ~50 ms of GPU spin while the calls queue up
        for i in range(warm):                  # untimed calls: clocks back up after the spin
            body(i)
        e0.record(self.stream)
        for i in range(n):
            body(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n   # us per call

    def back_to_back(self, fn, n):
        return self._bracket(fn, n)

    def cold(self, fn, n, prep=None):
        """Per-call time with a cache flush (and an optional prep) before every
        call: (flush; prep; call) x n minus (flush; prep) x n."""
        def with_call(i):
            self.flush()
            if prep:
                prep()
            fn(i)

        def without(i):
            self.flush()
            if prep:
                prep()
        t_all = self._bracket(with_call, n)
        t_base = self._bracket(without, n)
        if t_all - t_base > 0.0:
            return t_all - t_base
        # The difference can vanish under a profiler that serialises kernels
        # (counter collection); then report back-to-back calls, never zero.
        def call(i):
            if prep:
                prep()
            fn(i)
        return self._bracket(call, n)


def stream_rates(dev, timer, mib=2048, reps=10):
    """The device's practical streaming rates, measured now with the plain
    read and copy kernels of libstreamprobe.so (GB/s of bytes moved; the best
    of a few launch shapes), plus the rate of re-reading 64 MB that was just
    read (served by the Infinity Cache when it holds it)."""
    import ctypes
    import torch
    from long_context_verify_amd.build import PROBE_LIB_PATH
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    lib.probe_stream_read.restype = ctypes.c_int
    lib.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.probe_stream_copy.restype = ctypes.c_int
    lib.probe_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)

    def read(nbytes, grid, unroll, nt):
        def f(i):
            if lib.probe_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), grid, unroll, nt,
                                     stream) != 0:
                raise RuntimeError("probe_stream_read failed")
        f(0)
        return f

    def copy(grid, unroll):
        def f(i):
            if lib.probe_stream_copy(src.data_ptr(), dst.data_ptr(), n, grid, unroll,
                                     stream) != 0:
                raise RuntimeError("probe_stream_copy failed")
        f(0)
        return f
    best_r, cfg_r = 0.0, None
    for grid in (1024, 2048, 4096):
        for unroll in (8, 16):
            for nt in (0, 1):
                t = timer.back_to_back(read(n, grid, unroll, nt), reps)
                if n / t / 1e3 > best_r:
                    best_r, cfg_r = n / t / 1e3, (grid, unroll, nt)
    best_c, cfg_c = 0.0, None
    for grid in (1024, 2048, 4096):
        for unroll in (4, 8):
            t = timer.back_to_back(copy(grid, unroll), reps)
            if 2 * n / t / 1e3 > best_c:
                best_c, cfg_c = 2 * n / t / 1e3, (grid, unroll)
    small = 64 << 20
    t_small = timer.back_to_back(read(small, cfg_r[0], cfg_r[1], 0), reps * 5)
    del src, dst
    return {"read_GBps": best_r, "copy_GBps": best_c, "bytes": n,
            "cache_reread_GBps": small / t_small / 1e3,
            "how": (f"libstreamprobe.so plain read / copy kernels over {mib} MiB, best of "
                    f"launch shapes (read: {cfg_r[0]} work-groups x {cfg_r[1]} 4-KB steps, "
                    f"{'non-temporal' if cfg_r[2] else 'plain'} loads; copy: {cfg_c[0]} x "
                    f"{cfg_c[1]}), {reps} back-to-back calls between HIP events; "
                    f"cache_reread: the same read kernel over 64 MiB read just before")}


# ---------------------------------------------------------------------------
# Inputs
# ---------------------------------------------------------------------------
def build_inputs(cfg, dev, with_window=True):
    from workloads import make_attention_inputs, make_sample_inputs, make_window_inputs, random_tree
    att = make_attention_inputs(cfg.batch, cfg.hq, cfg.hkv, cfg.n_q, cfg.head_dim, cfg.kv_len,
                                dtype=cfg.dtype, seed=cfg.seed, device=dev)
    parent = random_tree(cfg.n_q) if cfg.tree else None
    win = None
    if cfg.window is not None and with_window:
        win = make_window_inputs(cfg.batch, cfg.hq, cfg.hkv, cfg.head_dim, cfg.window, cfg.sinks,
                                 [cfg.kv_len] * cfg.batch, dtype=cfg.dtype, seed=cfg.seed + 1,
                                 device=dev)
    sparent = parent if cfg.tree else None
    smp = make_sample_inputs(cfg.batch, cfg.n_nodes, cfg.vocab, sparent, cfg.target_std,
                             draft_noise_std=cfg.draft_noise_std, draft_std=cfg.draft_std,
                             seed=cfg.seed + 2, device=dev)
    return att, parent, win, smp


def sample_rows_read(n_nodes, parent):
    """Logit rows one sequence's sampling reads once: every target row + draft rows of internal nodes."""
    if parent is None:
        n_int = n_nodes - 1
    else:
        n_int = len(set(int(p) for p in parent[1:]))
    return n_nodes + n_int


def verify_bytes(cfg, esz):
    kv = 2 * cfg.batch * cfg.hkv * cfg.kv_len * cfg.head_dim * esz
    qo = 2 * cfg.batch * cfg.hq * cfg.n_q * cfg.head_dim * esz
    return kv + qo


# ---------------------------------------------------------------------------
# CPU baseline
# ---------------------------------------------------------------------------
def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            i = info[0]
            blas = f"{i.get('internal_api', '?')} {i.get('version', '?')} " \
                   f"({os.path.basename(i.get('filepath', '?'))})"
            threads = max(int(x.get("num_threads", 1)) for x in info)
    except Exception:  # pragma: no cover
        pass
    return model, blas, threads


def cpu_baseline(cfg, att, parent, win, smp, budget_s):
    """Time the fp64 oracle on a bounded sample of the step and scale it to the whole step."""
    from oracle.attention import verify_attention, window_attention
    from oracle.sample import spec_sample
    model, blas, threads = cpu_info()
    g = cfg.hq // cfg.hkv
    units = cfg.batch * cfg.hkv
    share = budget_s / 3.0
    # (1) verify attention: whole (sequence, kv head) units
    t_unit, n_unit = 0.0, 0
    while t_unit < share and n_unit < units:
        b, hk = divmod(n_unit, cfg.hkv)
        q = att["q"][b:b + 1, hk * g:(hk + 1) * g].cpu()
        k = att["k"][b:b + 1, hk:hk + 1].cpu()
        v = att["v"][b:b + 1, hk:hk + 1].cpu()
        t0 = time.perf_counter()
        verify_attention(q, k, v, [cfg.kv_len], parent)
        t_unit += time.perf_counter() - t0
        n_unit += 1
    t_verify = t_unit / n_unit * units
    # (2) window attention: whole sequences
    t_window, n_win = 0.0, 0
    if win is not None:
        t_w = 0.0
        while t_w < share / 2 and n_win < cfg.batch:
            b = n_win
            sl = slice(b, b + 1)
            args = [win[k][sl].cpu() for k in ("q", "hist_sink_k", "hist_sink_v",
                                               "hist_recent_k", "hist_recent_v")]
            t0 = time.perf_counter()
            window_attention(*args, [cfg.kv_len], cfg.window, cfg.sinks)
            t_w += time.perf_counter() - t0
            n_win += 1
        t_window = t_w / n_win * cfg.batch
    # (3) sampling: whole sequences
    t_s, n_seq = 0.0, 0
    while t_s < share and n_seq < cfg.batch:
        b = n_seq
        tl, dl, tk = (smp[k][b:b + 1].cpu() for k in ("target", "draft", "tokens"))
        t0 = time.perf_counter()
        spec_sample(tl, dl, tk, parent if cfg.tree else None, seed=1, offset=0)
        t_s += time.perf_counter() - t0
        n_seq += 1
    t_sample = t_s / n_seq * cfg.batch
    t_step = t_verify + t_window + t_sample
    drafts = cfg.batch * (cfg.n_nodes - 1)
    return {
        "value": drafts / t_step, "unit": "verified draft tokens/s", "cores": int(threads),
        "kind": "oracle", "cpu_model": model, "blas": blas,
        "sample": (f"{n_unit}/{units} verify units (sequence x kv head), {n_win}/{cfg.batch} "
                   f"window sequences, {n_seq}/{cfg.batch} sampling sequences of {cfg.name}; "
                   f"fp64 numpy, scaled to the whole step ({t_step:.2f} s/step)"),
        "ms_per_step": t_step * 1e3,
    }


# ---------------------------------------------------------------------------
# One workload's ops
# ---------------------------------------------------------------------------
class WorkloadOps:
    """Preallocated outputs and workspaces of one workload: the timed calls allocate nothing."""

    def __init__(self, L, cfg, dev, att, parent, win, smp, seed, page_size=0, siblings="first"):
        import torch
        self.L, self.cfg, self.att, self.parent, self.win, self.smp = L, cfg, att, parent, win, smp
        self.seed, self.page_size, self.siblings = seed, page_size, siblings
        B, Hq, Hkv, D, Lk, nq = cfg.batch, cfg.hq, cfg.hkv, cfg.head_dim, cfg.kv_len, cfg.n_q
        dt = att["q"].dtype
        self.out = torch.empty_like(att["q"])
        self.lse = torch.empty(B, Hq, nq, dtype=torch.float32, device=dev)
        self.ws_v = torch.zeros(max(L.verify_attention_workspace_bytes(B, Hq, Hkv, nq, D, Lk, dt),
                                    256), dtype=torch.uint8, device=dev)
        self.par_t = None if parent is None else torch.as_tensor(parent, dtype=torch.int32,
                                                                  device=dev)
        if win is not None:
            self.wout = torch.empty_like(win["q"])
            self.wlse = torch.empty(B, Hq, 1, dtype=torch.float32, device=dev)
            self.ws_w = torch.zeros(max(L.window_attention_workspace_bytes(
                B, Hq, Hkv, D, cfg.window, cfg.sinks, dt), 256), dtype=torch.uint8, device=dev)
        N, V = cfg.n_nodes, cfg.vocab
        self.s_out = {"out_tokens": torch.empty(B, N, dtype=torch.int32, device=dev),
                      "out_count": torch.empty(B, dtype=torch.int32, device=dev),
                      "out_path": torch.empty(B, N, dtype=torch.int32, device=dev),
                      "out_accept": torch.empty(B, N, dtype=torch.uint8, device=dev)}
        self.ws_s = torch.zeros(max(L.sample_workspace_bytes(B, N, V), 256), dtype=torch.uint8,
                                device=dev)
        if page_size:
            from workloads import make_paged_inputs
            self.pg = make_paged_inputs(att["k"], att["v"], att["kv_len"], page_size,
                                        seed=cfg.seed)
            self.ws_v = torch.zeros(max(L.verify_attention_paged_workspace_bytes(
                B, Hq, Hkv, nq, D, Lk, page_size, dt), 256), dtype=torch.uint8, device=dev)

    def verify(self, i=0):
        a, L = self.att, self.L
        if self.page_size:
            L.verify_attention_paged(a["q"], self.pg["k_pages"], self.pg["v_pages"],
                                     self.pg["block_table"], a["kv_len"], self.cfg.kv_len,
                                     parent=self.par_t, out=self.out, lse=self.lse,
                                     workspace=self.ws_v)
        else:
            L.verify_attention(a["q"], a["k"], a["v"], a["kv_len"], parent=self.par_t,
                               out=self.out, lse=self.lse, workspace=self.ws_v)

    def window(self, i=0):
        w = self.win
        self.L.window_attention(w["q"], w["k_ring"], w["v_ring"], w["k_sink"], w["v_sink"],
                                w["total_len"], out=self.wout, lse=self.wlse, workspace=self.ws_w)

    def sample(self, i=0):
        s = self.smp
        self.L.spec_sample(s["target"], s["draft"], s["tokens"],
                           parent=self.par_t if self.cfg.tree else None, seed=self.seed,
                           offset=i % (1 << 20), workspace=self.ws_s, siblings=self.siblings,
                           **self.s_out)

    def step_ops(self):
        ops = [("verify_attn", self.verify)]
        if self.win is not None:
            ops.append(("window_attn", self.window))
        ops.append(("sample", self.sample))
        return ops

    def verify_bytes(self):
        return verify_bytes(self.cfg, self.att["q"].element_size())

    def sample_bytes(self):
        rows = sample_rows_read(self.cfg.n_nodes, self.parent if self.cfg.tree else None)
        return self.cfg.batch * rows * self.cfg.vocab * self.smp["target"].element_size()


def op_figures(timer, ops, steps):
    """us / GB/s of the verify and sampling calls of one workload."""
    rep = {}
    t_v = timer.back_to_back(ops.verify, steps)
    vb = ops.verify_bytes()
    rep["verify_attn"] = {"us": t_v, "bytes": vb, "GBps": vb / t_v / 1e3,
                          "hbm_frac": vb / t_v / 1e3 / HBM_PEAK_GBPS,
                          "timing": "events around K back-to-back calls"
                          if vb >= BIG_OP_BYTES else
                          "events around K back-to-back calls (K/V partly cache-resident)"}
    sb = ops.sample_bytes()
    t_s = timer.cold(ops.sample, steps)
    t_sw = timer.back_to_back(ops.sample, steps)
    rep["sample"] = {"us": t_s, "us_warm": t_sw, "bytes": sb, "GBps": sb / t_s / 1e3,
                     "hbm_frac": sb / t_s / 1e3 / HBM_PEAK_GBPS,
                     "drafts_per_call": ops.cfg.batch * (ops.cfg.n_nodes - 1),
                     "timing": "K x (cache flush; call) minus K x flush, one event pair each; "
                               "us_warm: K back-to-back calls"}
    if ops.cfg.tree:
        flops = 4.0 * ops.cfg.batch * ops.cfg.hq * ops.cfg.n_q * ops.cfg.kv_len * ops.cfg.head_dim
        rep["verify_attn"]["mfma_TFLOPs"] = flops / (t_v * 1e-6) / 1e12
        rep["verify_attn"]["mfma_frac"] = rep["verify_attn"]["mfma_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
    return rep


def window_scaling(L, dev, timer, steps):
    """Draft window attention vs full-cache n_q = 1 attention as the context grows.

    The 8B/32K layer shape (batch 8, 32 q heads, 8 kv heads, head dim 128,
    bf16) with a 512-slot ring + 4 sinks: the window's cost stays flat while
    attention of one query over the whole cache grows with T.
    """
    import torch
    from workloads import make_attention_inputs, make_window_inputs
    B, Hq, Hkv, D, W, S = 8, 32, 8, 128, 512, 4
    rows = []
    win = make_window_inputs(B, Hq, Hkv, D, W, S, [W + S] * B, dtype="bf16", seed=77, device=dev)
    wout = torch.empty_like(win["q"])
    ws_w = torch.zeros(max(L.window_attention_workspace_bytes(B, Hq, Hkv, D, W, S,
                                                              torch.bfloat16), 256),
                       dtype=torch.uint8, device=dev)
    for T in (1024, 8192, 32768, 131072):
        tl = torch.full((B,), T, dtype=torch.int32, device=dev)

        def fwin(i):
            L.window_attention(win["q"], win["k_ring"], win["v_ring"], win["k_sink"],
                               win["v_sink"], tl, out=wout, workspace=ws_w, want_lse=False)
        fwin(0)
        t_w = timer.cold(fwin, steps)
        t_ww = timer.back_to_back(fwin, steps)
        att = make_attention_inputs(B, Hq, Hkv, 1, D, T, dtype="bf16", seed=78, device=dev)
        out = torch.empty_like(att["q"])
        ws_v = torch.zeros(max(L.verify_attention_workspace_bytes(B, Hq, Hkv, 1, D, T,
                                                                  torch.bfloat16), 256),
                           dtype=torch.uint8, device=dev)

        def ffull(i):
            L.verify_attention(att["q"], att["k"], att["v"], att["kv_len"], out=out,
                               workspace=ws_v, want_lse=False)
        ffull(0)
        kvb = 2 * B * Hkv * T * D * 2
        t_f = timer.back_to_back(ffull, steps) if kvb >= BIG_OP_BYTES else timer.cold(ffull, steps)
        rows.append({"T": T, "window_us": t_w, "window_us_warm": t_ww, "full_us": t_f,
                     "full_kv_bytes": kvb,
                     "window_kv_bytes": 2 * B * Hkv * min(T, W + S) * D * 2})
        del att, out, ws_v
        torch.cuda.empty_cache()
    return {"shape": "batch 8, 32 q heads / 8 kv heads, head dim 128, bf16; window 512 + 4 sinks",
            "timing": "window: K x (cache flush; call) minus K x flush; full: K back-to-back "
                      "calls when the cache exceeds 768 MB, else flushed like the window",
            "rows": rows}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the verification "
              "path is measured on a single MI355X and multi-GPU runs are not part of it.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_verify_amd as L
    from workloads import CONFIGS

    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L.lib()  # fail loudly if the library is missing
    timer = Timer(dev)
    if args.window_scaling_only:
        print(json.dumps({"window_scaling": window_scaling(L, dev, timer, min(args.steps, 30))}),
              flush=True)
        return
    log(f"[bench] building inputs for {cfg.name}")
    att, parent, win, smp = build_inputs(cfg, dev)
    if args.logits == "bf16":
        smp["target"] = smp["target"].to(torch.bfloat16)
        smp["draft"] = smp["draft"].to(torch.bfloat16)
    seed = 0x5EED0000 + cfg.seed
    ops = WorkloadOps(L, cfg, dev, att, parent, win, smp, seed, args.page_size, args.siblings)
    B, Hq, Hkv, D, Lk, nq = cfg.batch, cfg.hq, cfg.hkv, cfg.head_dim, cfg.kv_len, cfg.n_q
    N, V = cfg.n_nodes, cfg.vocab
    dt = att["q"].dtype
    esz = att["q"].element_size()
    step_ops = ops.step_ops()

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src_b = torch.ones(n, dtype=torch.uint8, device=dev)
        dst_b = torch.empty_like(src_b)
        for _ in range(3):
            dst_b.copy_(src_b)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 3 x {args.copy_probe_mib} MiB device-to-device copies")
        del src_b, dst_b

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        for _, f in step_ops:
            f(i)
    torch.cuda.synchronize()

    # (A) Headline: K whole steps back to back, host clock around a device sync.
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for _, f in step_ops:
            f(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # The same step with the Infinity Cache flushed before each one (events,
    # the flush's own time subtracted): at the chain workloads each step's
    # verify already streams far more than the cache holds, so the two agree.
    def whole_step(i):
        for _, f in step_ops:
            f(i)
    us_step_cold = timer.cold(whole_step, args.steps)

    # (B) Per-op device times.
    op_rep = op_figures(timer, ops, args.steps)
    if win is not None:
        keys = cfg.sinks + cfg.window
        wbytes = 2 * B * Hkv * keys * D * esz + 2 * B * Hq * D * esz
        t_w = timer.cold(ops.window, args.steps)
        op_rep["window_attn"] = {"us": t_w, "us_warm": timer.back_to_back(ops.window, args.steps),
                                 "bytes": wbytes, "GBps": wbytes / t_w / 1e3,
                                 "timing": op_rep["sample"]["timing"]}

    # Calls on either side of the step: the draft-step draw and the commit.
    d_tok = torch.empty(B, dtype=torch.int32, device=dev)
    d_lp = torch.empty(B, dtype=torch.float32, device=dev)
    ws_d = torch.zeros(max(L.draft_sample_workspace_bytes(B, V), 256), dtype=torch.uint8,
                       device=dev)

    def op_draft(i):
        # One draft step: the draw of node 1 from draft row 0 of every sequence.
        L.draft_sample(smp["draft"][:, 0], 1, seed=seed, offset=i, out_token=d_tok,
                       out_logprob=d_lp, workspace=ws_d)
    t_d = timer.cold(op_draft, args.steps)
    dbytes = B * V * smp["target"].element_size()
    op_rep["draft_sample"] = {"us": t_d, "us_warm": timer.back_to_back(op_draft, args.steps),
                              "bytes": dbytes, "GBps": dbytes / t_d / 1e3,
                              "timing": op_rep["sample"]["timing"]}

    # The commit updates lengths in place: each call is preceded by a restore
    # of the lengths, which the subtraction removes with the flush.
    kl_c = att["kv_len"].clone()
    tl_c = None if win is None else win["total_len"].clone()

    def prep_commit():
        kl_c.copy_(att["kv_len"])
        if tl_c is not None:
            tl_c.copy_(win["total_len"])

    def op_commit(i):
        L.kv_commit(att["k"], att["v"], kl_c, ops.s_out["out_count"], nq,
                    path=ops.s_out["out_path"] if cfg.tree else None, draft_total_len=tl_c,
                    draft_appended=nq - 1 if tl_c is not None else 0)
    ops.sample(0)
    t_c = timer.cold(op_commit, args.steps, prep=prep_commit)
    counts = ops.s_out["out_count"].cpu().numpy()
    moved = 0
    if cfg.tree:
        paths = ops.s_out["out_path"].cpu().numpy()
        for b in range(B):
            c = int(counts[b])
            j0 = next((j for j in range(c) if paths[b, j] != j), c)
            moved += c - j0
    op_rep["kv_commit"] = {"us": t_c, "bytes": 2 * 2 * moved * Hkv * D * esz,
                           "rows_moved": moved, "accepted_mean": float(counts.mean()),
                           "timing": "K x (cache flush; length restore; call) minus "
                                     "K x (flush; restore)"}
    log(f"[bench] per-op us: " + ", ".join(f"{k} {v['us']:.2f}" for k, v in op_rep.items()))

    rates = stream_rates(dev, timer)
    log(f"[bench] stream read {rates['read_GBps']:.0f} GB/s, copy {rates['copy_GBps']:.0f} GB/s, "
        f"64 MB re-read {rates['cache_reread_GBps']:.0f} GB/s")

    drafts = B * (N - 1)
    value = drafts / (ms_step / 1e3)
    v_rep = op_rep["verify_attn"]
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_flushed": us_step_cold / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt != torch.float32 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "kv_len": Lk, "block": "tree" if cfg.tree else "chain",
                   "gamma": nq - 1, "draft_window": cfg.window,
                   "sinks": cfg.sinks if cfg.window is not None else None,
                   "vocab": V, "logits": args.logits, "siblings": args.siblings,
                   "kv_layout": (f"paged, {args.page_size} keys per page"
                                 if args.page_size else "contiguous"),
                   "parallelism": "single-gpu"},
        "verify_attn_GBps": v_rep["GBps"],
        "verify_attn_hbm_frac": v_rep["hbm_frac"],
        "roofline": {
            "kernel": "spec_verify_attention",
            "bound": "hbm",
            "achieved": v_rep["GBps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": v_rep["hbm_frac"],
            "traffic": recorded_traffic(cfg.name),
            "frac_measured_peak": v_rep["GBps"] / rates["read_GBps"],
            "measured_peak": rates,
        },
        "roofline_sample": {
            "kernel": "spec_sample", "bound": "hbm", "achieved": op_rep["sample"]["GBps"],
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": op_rep["sample"]["hbm_frac"],
            "frac_measured_peak": op_rep["sample"]["GBps"] / rates["read_GBps"],
            "verified_drafts_per_s": op_rep["sample"]["drafts_per_call"]
            / (op_rep["sample"]["us"] * 1e-6),
        },
        "ops": op_rep,
    }
    if cfg.tree:
        # Wide query blocks sit near the MFMA ridge: co-report the dense bf16
        # rate of the same call (Q K^T and P V, 2 flop per multiply-add).
        res["roofline_mfma"] = {"kernel": "spec_verify_attention", "bound": "mfma",
                                "achieved": v_rep["mfma_TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": v_rep["mfma_frac"]}
    cpu = None
    if args.cpu_budget > 0:
        log("[bench] timing the oracle on a bounded sample (CPU)")
        cpu = cpu_baseline(cfg, att, parent, win, smp, args.cpu_budget)

    # Free the headline inputs before the extra runs.
    del ops, att, win, smp, step_ops
    torch.cuda.empty_cache()

    if not args.no_others:
        others = {}
        for name, ocfg in CONFIGS.items():
            if name == cfg.name or ocfg.dtype != "bf16":
                continue
            log(f"[bench] other workload {name}")
            oatt, opar, _, osmp = build_inputs(ocfg, dev, with_window=False)
            oops = WorkloadOps(L, ocfg, dev, oatt, opar, None, osmp, 0x5EED0000 + ocfg.seed)
            oops.verify(0)
            oops.sample(0)
            others[name] = op_figures(timer, oops, args.steps)
            del oops, oatt, osmp
            torch.cuda.empty_cache()
        res["workloads"] = others
    if not args.no_window_scaling:
        log("[bench] window scaling")
        res["window_scaling"] = window_scaling(L, dev, timer, min(args.steps, 30))
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
