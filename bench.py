#!/usr/bin/env python3
"""Benchmark of one speculative verification step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input,
shaped like an 8B-class GQA layer at 32K context (batch 8, 32 query heads,
8 KV heads, head dim 128, bf16, gamma = 4):

  1. spec_verify_attention  the gamma+1 = 5 block queries of every sequence
                            against its 32768-token KV cache (causal chain);
  2. spec_window_attention  one draft-step query against 4 sink tokens and a
                            512-slot ring (the MagicDec bounded draft cache);
  3. spec_sample            acceptance test + residual/bonus draw over a
                            128256-token vocabulary (5 target rows, 4 draft rows
                            per sequence).

All inputs are resident in HBM before the timed region.  The printed value
is verified draft tokens per second (batch * gamma per step).  Per-op times
come from HIP events recorded on the stream the library launches on (torch's
current stream); besides the three step ops they cover the calls on either
side of the step, spec_draft_sample (one draft-step draw) and spec_kv_commit
(keeping the accepted path), which are not part of the step.  The oracle
(fp64 numpy) is timed on a bounded sample of the same workload on the host
cores and reported as ``cpu_baseline``.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--page-size P] [--logits f32|bf16] [--siblings first|lossless]
                       [--cpu-budget SECONDS] [--copy-probe-mib MIB]
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


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["long_context_verify_amd/csrc/attention.hip",
                  "long_context_verify_amd/csrc/spec_common.hpp",
                  "long_context_verify_amd/csrc/spec_internal.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_attn_llama8b_32k_hbm_counters.txt")


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
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
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
    p.add_argument("--workload", default="llama8b_32k_chain")
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
    return p.parse_args()


def build_inputs(cfg, dev):
    from workloads import (chain_parent, make_attention_inputs, make_sample_inputs,
                           make_window_inputs, random_tree)
    att = make_attention_inputs(cfg.batch, cfg.hq, cfg.hkv, cfg.n_q, cfg.head_dim, cfg.kv_len,
                                dtype=cfg.dtype, seed=cfg.seed, device=dev)
    parent = random_tree(cfg.n_q) if cfg.tree else None
    win = None
    if cfg.window is not None:
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


def cpu_baseline(cfg, att, parent, win, smp, budget_s):
    """Time the fp64 oracle on a bounded sample of the step and scale it to the whole step."""
    import torch
    from oracle.attention import verify_attention, window_attention
    from oracle.sample import spec_sample
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
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
        "kind": "oracle",
        "sample": (f"{n_unit}/{units} verify units (sequence x kv head), {n_win}/{cfg.batch} "
                   f"window sequences, {n_seq}/{cfg.batch} sampling sequences; fp64 numpy, "
                   f"scaled to the whole step ({t_step:.2f} s/step)"),
        "ms_per_step": t_step * 1e3,
    }


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
    log(f"[bench] building inputs for {cfg.name}")
    att, parent, win, smp = build_inputs(cfg, dev)
    if args.logits == "bf16":
        smp["target"] = smp["target"].to(torch.bfloat16)
        smp["draft"] = smp["draft"].to(torch.bfloat16)
    lsz = smp["target"].element_size()
    B, Hq, Hkv, D, Lk, nq = cfg.batch, cfg.hq, cfg.hkv, cfg.head_dim, cfg.kv_len, cfg.n_q
    dt = att["q"].dtype
    esz = att["q"].element_size()

    # Preallocated outputs and workspaces: the timed loop allocates nothing.
    out = torch.empty_like(att["q"])
    lse = torch.empty(B, Hq, nq, dtype=torch.float32, device=dev)
    ws_v = torch.zeros(max(L.verify_attention_workspace_bytes(B, Hq, Hkv, nq, D, Lk, dt), 256),
                       dtype=torch.uint8, device=dev)
    par_t = None if parent is None else torch.as_tensor(parent, dtype=torch.int32, device=dev)
    if win is not None:
        wout = torch.empty_like(win["q"])
        wlse = torch.empty(B, Hq, 1, dtype=torch.float32, device=dev)
        ws_w = torch.zeros(max(L.window_attention_workspace_bytes(B, Hq, Hkv, D, cfg.window,
                                                                  cfg.sinks, dt), 256),
                           dtype=torch.uint8, device=dev)
    N, V = cfg.n_nodes, cfg.vocab
    s_out = {"out_tokens": torch.empty(B, N, dtype=torch.int32, device=dev),
             "out_count": torch.empty(B, dtype=torch.int32, device=dev),
             "out_path": torch.empty(B, N, dtype=torch.int32, device=dev),
             "out_accept": torch.empty(B, N, dtype=torch.uint8, device=dev)}
    ws_s = torch.zeros(max(L.sample_workspace_bytes(B, N, V), 256), dtype=torch.uint8, device=dev)
    seed = 0x5EED0000 + cfg.seed

    if args.page_size:
        from workloads import make_paged_inputs
        pg = make_paged_inputs(att["k"], att["v"], att["kv_len"], args.page_size, seed=cfg.seed)
        ws_v = torch.zeros(max(L.verify_attention_paged_workspace_bytes(
            B, Hq, Hkv, nq, D, Lk, args.page_size, dt), 256), dtype=torch.uint8, device=dev)

    def op_verify():
        if args.page_size:
            L.verify_attention_paged(att["q"], pg["k_pages"], pg["v_pages"], pg["block_table"],
                                     att["kv_len"], Lk, parent=par_t, out=out, lse=lse,
                                     workspace=ws_v)
        else:
            L.verify_attention(att["q"], att["k"], att["v"], att["kv_len"], parent=par_t,
                               out=out, lse=lse, workspace=ws_v)

    def op_window():
        L.window_attention(win["q"], win["k_ring"], win["v_ring"], win["k_sink"], win["v_sink"],
                           win["total_len"], out=wout, lse=wlse, workspace=ws_w)

    def op_sample(i):
        L.spec_sample(smp["target"], smp["draft"], smp["tokens"], parent=par_t if cfg.tree else None,
                      seed=seed, offset=i, workspace=ws_s, siblings=args.siblings, **s_out)

    ops = [("verify_attn", lambda i: op_verify())]
    if win is not None:
        ops.append(("window_attn", lambda i: op_window()))
    ops.append(("sample", op_sample))

    # The commit after sampling updates lengths in place, so it is timed on
    # its own (not part of the step) with the lengths restored before each
    # call, outside the timed bracket.
    kl_c = att["kv_len"].clone()
    tl_c = None if win is None else win["total_len"].clone()

    def prep_commit():
        kl_c.copy_(att["kv_len"])
        if tl_c is not None:
            tl_c.copy_(win["total_len"])

    d_tok = torch.empty(B, dtype=torch.int32, device=dev)
    d_lp = torch.empty(B, dtype=torch.float32, device=dev)
    ws_d = torch.zeros(max(L.draft_sample_workspace_bytes(B, V), 256), dtype=torch.uint8,
                       device=dev)

    def op_draft(i):
        # One draft step: the draw of node 1 from draft row 0 of every sequence.
        L.draft_sample(smp["draft"][:, 0], 1, seed=seed, offset=i, out_token=d_tok,
                       out_logprob=d_lp, workspace=ws_d)

    def op_commit(i):
        L.kv_commit(att["k"], att["v"], kl_c, s_out["out_count"], nq,
                    path=s_out["out_path"] if cfg.tree else None, draft_total_len=tl_c,
                    draft_appended=nq - 1 if tl_c is not None else 0)

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
        for _, f in ops:
            f(i)
    torch.cuda.synchronize()

    # (A) Headline: K whole steps back to back, host clock around a device sync.
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        for _, f in ops:
            f(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # (B) Per-op device time from HIP events on the stream the library launches
    # on (torch's current stream).  Everything is queued behind a GPU sleep so
    # host launch latency cannot leak into the bracketed time.  An op whose
    # inputs exceed the 256 MB Infinity Cache runs K times back to back between
    # one pair of events (its inputs come from HBM every time).  Smaller ops
    # get one pair per call, with a 512 MB read of an unrelated buffer between
    # calls (outside the brackets) so every call reads its inputs from HBM and
    # leaves no dirty lines to write back.
    stream = torch.cuda.current_stream(dev)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    op_bytes_in = {"verify_attn": att["k"].numel() * esz * 2,
                   "window_attn": 0 if win is None else
                   (win["k_ring"].numel() + win["k_sink"].numel()) * esz * 2,
                   "sample": smp["target"].numel() * 2 * lsz,
                   "draft_sample": B * V * lsz,
                   "kv_commit": 0}
    op_us = {}
    preps = {"kv_commit": prep_commit}
    for name, f in ops + [("draft_sample", op_draft), ("kv_commit", op_commit)]:
        big = op_bytes_in[name] >= (768 << 20)
        n_pairs = 1 if big else args.steps
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(n_pairs)]
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * 0.05))           # ~50 ms of GPU spin while we enqueue
        if big:
            pairs[0][0].record(stream)
            for i in range(args.steps):
                f(args.warmup + args.steps + i)
            pairs[0][1].record(stream)
        else:
            for i, (e0, e1) in enumerate(pairs):
                flush.amax()
                if name in preps:
                    preps[name]()
                e0.record(stream)
                f(args.warmup + args.steps + i)
                e1.record(stream)
        torch.cuda.synchronize()
        per_call = [a.elapsed_time(b) * 1e3 for a, b in pairs]
        op_us[name] = float(np.sum(per_call) / args.steps)
    log(f"[bench] per-op mean us: {op_us}")

    # Algorithmic bytes per call.
    kv_bytes = 2 * B * Hkv * Lk * D * esz
    qo_bytes = 2 * B * Hq * nq * D * esz
    verify_bytes = kv_bytes + qo_bytes
    ops_report = {"verify_attn": {
        "us": op_us["verify_attn"], "bytes": verify_bytes,
        "GBps": verify_bytes / op_us["verify_attn"] / 1e3,
    }}
    ops_report["verify_attn"]["hbm_frac"] = ops_report["verify_attn"]["GBps"] / HBM_PEAK_GBPS
    if win is not None:
        keys = cfg.sinks + cfg.window
        wbytes = 2 * B * Hkv * keys * D * esz + 2 * B * Hq * D * esz
        ops_report["window_attn"] = {"us": op_us["window_attn"], "bytes": wbytes,
                                     "GBps": wbytes / op_us["window_attn"] / 1e3}
    srows = sample_rows_read(N, parent if cfg.tree else None)
    sbytes = B * srows * V * lsz
    ops_report["sample"] = {"us": op_us["sample"], "bytes": sbytes,
                            "GBps": sbytes / op_us["sample"] / 1e3}
    ops_report["sample"]["hbm_frac"] = ops_report["sample"]["GBps"] / HBM_PEAK_GBPS
    dbytes = B * V * lsz
    ops_report["draft_sample"] = {"us": op_us["draft_sample"], "bytes": dbytes,
                                  "GBps": dbytes / op_us["draft_sample"] / 1e3}
    # Commit: K and V rows of the accepted path read and written back, from the
    # first node that is not already in place (a chain moves nothing).
    counts = s_out["out_count"].cpu().numpy()
    moved = 0
    if cfg.tree:
        paths = s_out["out_path"].cpu().numpy()
        for b in range(B):
            c = int(counts[b])
            j0 = next((j for j in range(c) if paths[b, j] != j), c)
            moved += c - j0
    cbytes = 2 * 2 * moved * Hkv * D * esz
    ops_report["kv_commit"] = {"us": op_us["kv_commit"], "bytes": cbytes,
                               "rows_moved": moved, "accepted_mean": float(counts.mean())}
    for name, rep in ops_report.items():
        rep["timing"] = ("events around K back-to-back calls"
                         if op_bytes_in[name] >= (768 << 20) else
                         "events around each call, cache flushed between calls")

    drafts = B * (N - 1)
    value = drafts / (ms_step / 1e3)
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt != torch.float32 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "kv_len": Lk, "block": "tree" if cfg.tree else "chain",
                   "gamma": nq - 1, "draft_window": cfg.window, "sinks": cfg.sinks,
                   "vocab": V, "logits": args.logits, "siblings": args.siblings, "kv_layout": (f"paged, {args.page_size} keys per page"
                                             if args.page_size else "contiguous"),
                   "parallelism": "single-gpu"},
        "verify_attn_GBps": ops_report["verify_attn"]["GBps"],
        "verify_attn_hbm_frac": ops_report["verify_attn"]["hbm_frac"],
        "roofline": {
            "kernel": "spec_verify_attention",
            "bound": "hbm",
            "achieved": ops_report["verify_attn"]["GBps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": ops_report["verify_attn"]["hbm_frac"],
            "traffic": recorded_traffic(cfg.name),
        },
        "ops": ops_report,
    }
    if cfg.tree:
        # Wide query blocks sit near the MFMA ridge: co-report the dense bf16
        # rate of the same call (Q K^T and P V, 2 flop per multiply-add).
        flops = 4.0 * B * Hq * nq * Lk * D
        tflops = flops / (op_us["verify_attn"] * 1e-6) / 1e12
        res["roofline_mfma"] = {"kernel": "spec_verify_attention", "bound": "mfma",
                                "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS}
    if args.cpu_budget > 0:
        log("[bench] timing the oracle on a bounded sample (CPU)")
        res["cpu_baseline"] = cpu_baseline(cfg, att, parent, win, smp, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
