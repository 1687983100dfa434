#!/usr/bin/env python3
"""Decode-step throughput of the TokenSelect hot path on one MI355X.

Workload (default): one decode step of one layer at the Qwen2-7B attention
shape (28 query / 4 KV heads, head_dim 128, bf16 KV) over N = 131072 cached
tokens, batch 1, top-k 2048, 1% heavy keys. theta = 1.0 forces a full
selection on every step (cos <= 1 never exceeds it), so each step runs the
whole path: Selection-Cache check, K-scan scoring, soft vote, radix top-k,
sparse attention over the gathered rows, combine and state update.

Inputs are resident in HBM before timing starts. The step rotates over
`--kv-copies` identical copies of K/V so the 256 MB Infinity Cache cannot
serve the 134 MB K-scan from the previous step.

One JSON line on stdout:
  value          decode steps/s over exactly --steps miss steps (wall clock
                 between synchronizations)
  roofline       the K-scan kernel's algorithmic bytes / its average duration,
                 measured with HIP events around each of its launches on its
                 own stream (ts_profile_*), against MI355X's 8 TB/s and
                 against the read bandwidth measured on the box; with it the
                 K-scan + gather figure (both kernels' bytes over their time)
  cpu_baseline   the fp64 oracle timed on this host's cores on a bounded
                 sample of the same workload (plus one-thread times of the
                 tiny and 32K workloads)
  extra          per-step median / p10 / p90 over at least 100 event-timed
                 steps, eager and replayed from a HIP graph; hit steps; every
                 other workload (tiny fp32, 32K, 4 x 128K, the 256-step paged
                 selection-cache run split into hit and miss steps, the
                 512 x 65536 prefill chunk, Quest pages, the dense baseline,
                 a 28-layer decode loop); the GPU clock
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM bytes of the K-scan kernel from two rocprofv3 counter runs, scaled by a
# plain copy kernel of known size; valid only for the kernel sources it names
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_pass1_qwen2-7b_n131072_traffic.txt")
KSCAN_SOURCES = ["sparse_kv_cache_ts_amd/csrc/score.hip", "sparse_kv_cache_ts_amd/csrc/ts_device.h",
                 "sparse_kv_cache_ts_amd/csrc/ts_internal.h"]


def _die_multi_gpu(n):
    print(f"bench.py measures one GPU; --gpus {n} is not supported (this path has no "
          f"multi-GPU mode: each GPU would score and select its own sequences)", file=sys.stderr)
    sys.exit(2)


def kscan_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KSCAN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """Measured HBM bytes per K-scan launch, or None when the kernel changed since."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for ln in fh:
                if ":" in ln and not ln.startswith(" "):
                    a, b = ln.split(":", 1)
                    kv[a.strip()] = b.strip()
        if kv.get("kernel_sources_sha256_16") != kscan_source_hash():
            return None
        return int(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def calibrate_copy(nbytes=512 << 20, reps=5):
    """A plain elementwise copy of known size, for scaling HBM byte counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "launches": reps}), flush=True)


def measure_prefill(ts, W, reps=10, warmup=3):
    """512-query chunk over 65536 keys: soft votes (two MFMA passes) and per-row top-k."""
    import torch
    cfg = W.PREFILL_64K
    x = W.gen_prefill(cfg, device="cuda")
    q0 = x["q_pos0"]
    votes = torch.empty(cfg.chunk, cfg.n_ctx, dtype=torch.float32, device="cuda")
    idx = torch.empty(cfg.chunk, cfg.k, dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k, votes=votes, idx=idx)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k, votes=votes, idx=idx)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    ts.profile_reset()
    ts.profile_enable(True)
    for _ in range(reps):
        ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k, votes=votes, idx=idx)
    torch.cuda.synchronize()
    ts.profile_enable(False)
    kern = {n: (c, ms) for n, (c, ms) in ts.profile_read().items() if c}
    # each query then attends over its own selection
    out = torch.empty(cfg.chunk, cfg.num_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
    aws = ts.Workspace()
    for _ in range(warmup):
        ts.sparse_attend_prefill(x["q"], x["k_cache"], x["v_cache"], q0, idx, out=out, ws=aws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        ts.sparse_attend_prefill(x["q"], x["k_cache"], x["v_cache"], q0, idx, out=out, ws=aws)
    torch.cuda.synchronize()
    att_us = 1e6 * (time.perf_counter() - t0) / reps
    visible = sum(q0 + i + 1 for i in range(cfg.chunk))
    flop = 2.0 * cfg.num_q_heads * cfg.head_dim * visible          # one Q.K^T product
    t_lse = kern["prefill_lse"][1] / reps * 1e-3                   # pass 1 + merge
    t_vote = kern["prefill_votes"][1] / reps * 1e-3
    # pass 1 and pass 2 each evaluate every visible product once
    mfma_tflops = 2 * flop / (t_lse + t_vote) / 1e12
    del x, votes, idx, out
    torch.cuda.empty_cache()
    return {"workload": "512 queries x 65536 keys, 32/8 heads, d=128, bf16, top-k 4096",
            "us_per_chunk": round(1e6 * wall, 1),
            "scoring_us": round(1e6 * (t_lse + t_vote), 1),
            "kernels_us": {n: round(1e3 * ms / reps, 1) for n, (c, ms) in kern.items()},
            "sparse_attention_us": round(att_us, 1),
            "gathered_kv_bytes": cfg.chunk * cfg.k * 2 * cfg.num_kv_heads * cfg.head_dim * 2,
            "qkt_gflop_per_pass": round(flop / 1e9, 1),
            "mfma_tflops": round(mfma_tflops, 1),
            "mfma_frac": round(mfma_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}


def measure_dense(ts, W, cfg, steps, warmup, copies):
    """Full softmax attention over every cached token (the method's comparison arm)."""
    import torch
    x = W.gen_decode(cfg, device="cuda")
    Ks = [x["k_cache"]] + [x["k_cache"].clone() for _ in range(copies - 1)]
    Vs = [x["v_cache"]] + [x["v_cache"].clone() for _ in range(copies - 1)]
    out = torch.empty(cfg.batch, cfg.num_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
    ws = ts.Workspace()
    for i in range(warmup):
        ts.dense_attend(x["q"], Ks[i % copies], Vs[i % copies], x["seq_lens"], out=out, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ts.dense_attend(x["q"], Ks[i % copies], Vs[i % copies], x["seq_lens"], out=out, ws=ws)
    torch.cuda.synchronize()
    us = 1e6 * (time.perf_counter() - t0) / steps
    kv = 2 * cfg.batch * cfg.seq_len * kv_bytes_per_token(cfg)
    del Ks, Vs, x
    torch.cuda.empty_cache()
    return {"us_per_call": round(us, 2), "kv_bytes": kv, "GBps": round(kv / (us * 1e-6) / 1e9, 1),
            "us_at_hbm_peak": round(kv / (HBM_PEAK_GBPS * 1e3), 2)}


def kv_bytes_per_token(cfg) -> int:
    return cfg.num_kv_heads * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4)


def _pct(xs, q):
    ys = sorted(xs)
    if not ys:
        return None
    i = min(len(ys) - 1, max(0, int(round(q * (len(ys) - 1)))))
    return ys[i]


def step_stats(us):
    """median / p10 / p90 / mean of per-step times (us)."""
    return {"median": round(_pct(us, 0.5), 2), "p10": round(_pct(us, 0.1), 2),
            "p90": round(_pct(us, 0.9), 2), "mean": round(sum(us) / len(us), 2), "n": len(us)}


def measure_decode(ts, W, cfg, steps, warmup, copies, theta, profile, tag, nstat=100, graph=False):
    """Decode steps of one layer at `cfg` (selection every step with theta=1).

    * `steps` steps timed on the wall clock between synchronizations (the
      figure bench.py reports as its value);
    * max(nstat, steps) steps each bracketed by HIP events on the stream:
      median / p10 / p90 of the per-step time;
    * with `profile`, per-kernel times from the library's own events;
    * with `graph`, `copies` steps (one per K/V copy) captured in one HIP
      graph and replayed: the per-step time without host launches.
    K/V rotate over `copies` identical copies so that the Infinity Cache
    cannot serve a step's reads from the step before."""
    import torch

    x = W.gen_decode(cfg, device="cuda")
    Ks = [x["k_cache"]] + [x["k_cache"].clone() for _ in range(copies - 1)]
    Vs = [x["v_cache"]] + [x["v_cache"].clone() for _ in range(copies - 1)]
    q, lens = x["q"], x["seq_lens"]
    B, Hq, d, k = cfg.batch, cfg.num_q_heads, cfg.head_dim, cfg.k
    cache = ts.SelCache(B, Hq, d, k)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, k, dtype=torch.int32, device="cuda")
    hit = torch.empty(B, dtype=torch.int32, device="cuda")

    def step(i):
        c = i % copies
        cache.decode_step(q, Ks[c], Vs[c], lens, theta, out=out, idx_out=idx, hit_out=hit)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    hits = int(hit.sum().item())
    res = {"tag": tag, "wall_s": wall, "ms_per_step": 1e3 * wall / steps,
           "steps_per_s": steps / wall, "last_step_hits": hits}

    # per-step event timing
    n = max(nstat, steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    us = [1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
    res["step_us"] = step_stats(us)

    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(copies):
                step(c)
        g.replay()
        torch.cuda.synchronize()
        reps = max(2, n // copies)
        gv = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        gv[0].record()
        for r in range(reps):
            g.replay()
            gv[r + 1].record()
        torch.cuda.synchronize()
        gus = [1e3 * gv[r].elapsed_time(gv[r + 1]) / copies for r in range(reps)]
        res["graph_step_us"] = step_stats(gus)
        del g

    if profile:
        ts.profile_reset()
        ts.profile_enable(True)
        t1 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        res["profiled_ms_per_step"] = 1e3 * (time.perf_counter() - t1) / steps
        ts.profile_enable(False)
        kern = ts.profile_read()
        res["kernels_us"] = {n_: 1e3 * ms / c for n_, (c, ms) in kern.items() if c}
        res["kernel_launches_per_step"] = {n_: c / steps for n_, (c, ms) in kern.items() if c}
    cache.close()
    del Ks, Vs
    torch.cuda.empty_cache()
    return res, x


def measure_loop(ts, W, cfg, layers, tokens, warmup):
    """The decode loop of a model with `layers` attention layers: per token and
    layer, append the new K/V row, then one decode step (selection every step)
    with that layer's own selection-cache state. Eager launches vs the same
    token captured once as a HIP graph and replayed."""
    import torch
    x = W.gen_decode(cfg, device="cuda")
    B, Hq, Hkv, d, N, k = (cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                           cfg.seq_len, cfg.k)
    cap = N + 2 * (warmup + tokens) + 8
    dt = x["k_cache"].dtype
    L = []
    for _ in range(layers):
        kc = torch.empty(B, cap, Hkv, d, dtype=dt, device="cuda")
        vc = torch.empty(B, cap, Hkv, d, dtype=dt, device="cuda")
        kc[:, :N] = x["k_cache"]
        vc[:, :N] = x["v_cache"]
        L.append({"k": kc, "v": vc, "lens": x["seq_lens"].clone(),
                  "kn": torch.randn(B, Hkv, d, device="cuda").to(dt),
                  "vn": torch.randn(B, Hkv, d, device="cuda").to(dt),
                  "cache": ts.SelCache(B, Hq, d, k),
                  "out": torch.empty(B, Hq, d, dtype=torch.float32, device="cuda"),
                  "idx": torch.empty(B, k, dtype=torch.int32, device="cuda"),
                  "hit": torch.empty(B, dtype=torch.int32, device="cuda")})
    q = x["q"]
    lay = ts.make_layout(q, L[0]["k"])
    for l in L:
        l["cache"].ws.get(l["cache"].workspace_size(lay, B), q.device)

    def token():
        for l in L:
            ts.append_kv(l["kn"], l["vn"], l["k"], l["v"], l["lens"])
            l["cache"].decode_step(q, l["k"], l["v"], l["lens"], 1.0, out=l["out"],
                                   idx_out=l["idx"], hit_out=l["hit"])

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / n

    eager_ms = timed(token, tokens)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        token()
    graph_ms = timed(graph.replay, tokens)
    final = [int(l["lens"][0].item()) for l in L]
    for l in L:
        l["cache"].close()
    del L, graph
    torch.cuda.empty_cache()
    return {"workload": f"{layers} layers x (append K/V + decode step), {cfg.name}, N={N} "
                        f"growing by one per token, top-k {k}, selection every step",
            "layers": layers, "tokens": tokens, "eager_ms_per_token": round(eager_ms, 4),
            "graph_ms_per_token": round(graph_ms, 4),
            "graph_tokens_per_s": round(1e3 / graph_ms, 2),
            "graph_speedup": round(eager_ms / graph_ms, 3),
            "us_per_layer_graph": round(1e3 * graph_ms / layers, 2),
            "final_len": final[0]}


def measure_quest(ts, W, steps, warmup):
    """Quest-style page selection on the paged selection-cache workload (8
    sequences of 16K..256K tokens, 32/8 heads, page 16): per step the last
    page's extremes, page scores + top-256 pages per KV head, and attention
    over those pages. Next to it, one TokenSelect step with selection on the
    same KV (theta = 1), for scale."""
    import torch
    cfg = W.SELCACHE_RUN
    x = W.gen_run(cfg, device="cuda")
    q, lens, pt = x["queries"][0], x["seq_lens"], x["page_table"]
    kp, vp = x["k_pool"], x["v_pool"]
    B, Hq, Hkv, d, P = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    k_pages = cfg.k // P
    meta = ts.quest_meta(kp, pt, lens)
    pidx = torch.empty(B, Hkv, k_pages, dtype=torch.int32, device="cuda")
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    ws_s, ws_a = ts.Workspace(), ts.Workspace()

    def step():
        ts.quest_meta(kp, pt, lens, meta=meta, last_page_only=True)
        ts.quest_select(q, kp, meta, pt, lens, k_pages, page_idx=pidx, ws=ws_s)
        ts.quest_attend(q, kp, vp, pt, lens, pidx, out=out, ws=ws_a)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    us = 1e6 * (time.perf_counter() - t0) / steps
    ts.profile_reset()
    ts.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ts.profile_enable(False)
    kern = {n: round(1e3 * ms / c, 2) for n, (c, ms) in ts.profile_read().items() if c}
    n_list = lens.tolist()
    pages = [-(-n // P) for n in n_list]
    esz = 2
    meta_bytes = sum(pages) * Hkv * 2 * d * esz
    gathered = sum(min(k_pages, pg) * P for pg in pages) * Hkv * d * esz * 2
    kscan_bytes = sum(n_list) * Hkv * d * esz
    # TokenSelect on the same KV, selection every step
    cache = ts.SelCache(B, Hq, d, cfg.k)
    o2 = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        cache.decode_step(q, kp, vp, lens, 1.0, page_table=pt, out=o2, want_idx=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        cache.decode_step(q, kp, vp, lens, 1.0, page_table=pt, out=o2, want_idx=False)
    torch.cuda.synchronize()
    ts_us = 1e6 * (time.perf_counter() - t0) / steps
    # the same query again at theta = 0.9: every step after the first reuses the selection
    for _ in range(warmup):
        cache.decode_step(q, kp, vp, lens, 0.9, page_table=pt, out=o2, want_idx=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        cache.decode_step(q, kp, vp, lens, 0.9, page_table=pt, out=o2, want_idx=False)
    torch.cuda.synchronize()
    ts_hit_us = 1e6 * (time.perf_counter() - t0) / steps
    hits, _ = cache.stats(B)
    cache.close()
    t_score = kern.get("quest_score", float("nan"))
    del x, kp, vp, meta
    torch.cuda.empty_cache()
    return {"workload": f"{cfg.name}: {B} paged sequences, {sum(n_list)} tokens, {Hq}/{Hkv} heads, "
                        f"d={d}, bf16, page {P}, top-{k_pages} pages per KV head",
            "us_per_step": round(us, 2), "kernels_us": kern,
            "meta_bytes": meta_bytes, "gathered_kv_bytes": gathered,
            "page_score_GBps": round(meta_bytes / (t_score * 1e-6) / 1e9, 1),
            "page_score_hbm_frac": round(meta_bytes / (t_score * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "tokenselect_selection_step_us": round(ts_us, 2),
            "tokenselect_hit_step_us": round(ts_hit_us, 2),
            "tokenselect_hits": hits,
            "tokenselect_kscan_bytes": kscan_bytes}


def measure_selcache_run(ts, W):
    """The selection-cache decode run as a whole: 256 steps over 8 paged
    sequences of 16K..256K tokens (32/8 heads, d=128, bf16, page 16, top-4096)
    with slowly drifting queries and a fresh random query every 32 steps,
    theta = 0.9, the stored query compared with the previous step's. Every
    step is bracketed by HIP events; steps where some sequence missed are the
    run's miss steps (there selection runs), the others hit steps."""
    import torch
    cfg = W.SELCACHE_RUN
    x = W.gen_run(cfg, device="cuda")
    qs, lens, pt = x["queries"], x["seq_lens"], x["page_table"]
    kp, vp = x["k_pool"], x["v_pool"]
    B, Hq, d = cfg.batch, cfg.num_q_heads, cfg.head_dim
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    hit_steps = torch.empty(cfg.steps, B, dtype=torch.int32, device="cuda")

    def run(events):
        cache = ts.SelCache(B, Hq, d, cfg.k)
        if events:
            events[0].record()
        for t in range(cfg.steps):
            cache.decode_step(qs[t], kp, vp, lens, cfg.theta, page_table=pt, out=out,
                              hit_out=hit_steps[t], want_idx=False)
            if events:
                events[t + 1].record()
        torch.cuda.synchronize()
        return cache

    run(None).close()                                # warm-up run
    t0 = time.perf_counter()
    cache = run(None)
    wall = time.perf_counter() - t0
    cache.close()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(cfg.steps + 1)]
    cache = run(ev)
    hits, misses = cache.stats(B)
    cache.close()
    us = [1e3 * ev[t].elapsed_time(ev[t + 1]) for t in range(cfg.steps)]
    hs = hit_steps.cpu().tolist()
    # the same run replayed from one HIP graph: the cache reset, then the 256
    # steps, captured once (after an eager step that sizes the workspace); the
    # replay's decisions must be the eager run's
    cache = ts.SelCache(B, Hq, d, cfg.k)
    cache.decode_step(qs[0], kp, vp, lens, cfg.theta, page_table=pt, out=out,
                      hit_out=hit_steps[0], want_idx=False)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cache.reset()
        for t in range(cfg.steps):
            cache.decode_step(qs[t], kp, vp, lens, cfg.theta, page_table=pt, out=out,
                              hit_out=hit_steps[t], want_idx=False)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_us = 1e3 * g0.elapsed_time(g1) / cfg.steps
    graph_same = hit_steps.cpu().tolist() == hs
    del graph
    cache.close()
    hit_us = [u for u, h in zip(us, hs) if all(h)]
    miss_us = [u for u, h in zip(us, hs) if not all(h)]
    n_list = lens.tolist()
    bpt = cfg.num_kv_heads * d * 2
    gathered = sum(min(cfg.k, n) for n in n_list) * bpt * 2
    kscan = sum(n_list) * bpt
    res = {"workload": f"{cfg.name}: {cfg.steps} steps, {B} paged sequences of "
                       f"{cfg.min_len}..{cfg.max_len} tokens ({sum(n_list)} in all), "
                       f"{Hq}/{cfg.num_kv_heads} heads, d={d}, bf16, page {cfg.page_size}, "
                       f"top-{cfg.k}, theta {cfg.theta}, a fresh query every {cfg.jump_every} steps",
           "us_per_step": round(1e6 * wall / cfg.steps, 2),
           "event_us_per_step": step_stats(us),
           "hit_step_us": step_stats(hit_us) if hit_us else None,
           "miss_step_us": step_stats(miss_us) if miss_us else None,
           "graph_us_per_step": round(graph_us, 2), "graph_decisions_match_eager": graph_same,
           "hits": hits, "misses": misses,
           "hit_step_gathered_bytes": gathered, "miss_step_kscan_bytes": kscan}
    if hit_us:
        res["hit_step_GBps"] = round(gathered / (_pct(hit_us, 0.5) * 1e-6) / 1e9, 1)
    run_bytes = (len(miss_us) * (kscan + gathered) + len(hit_us) * gathered) / cfg.steps
    res["run_avg_algorithmic_bytes_per_step"] = int(run_bytes)
    res["run_avg_hbm_frac"] = round(run_bytes / (1e-6 * sum(us) / len(us)) / 1e9 / HBM_PEAK_GBPS, 4)
    del x, kp, vp
    torch.cuda.empty_cache()
    return res


def decode_bytes(cfg):
    """Algorithmic bytes of one decode step with selection: K scanned once,
    plus the gathered K and V rows of the selection."""
    bpt = kv_bytes_per_token(cfg)
    kscan = cfg.batch * cfg.seq_len * bpt
    gather = cfg.batch * min(cfg.k, cfg.seq_len) * bpt * 2
    return kscan, gather


def config_entry(cfg, r, read_peak):
    kscan, gather = decode_bytes(cfg)
    med = r["step_us"]["median"]
    e = {"batch": cfg.batch, "seq_len": cfg.seq_len, "k": cfg.k,
         "heads": f"{cfg.num_q_heads}/{cfg.num_kv_heads}", "head_dim": cfg.head_dim,
         "dtype": cfg.dtype, "steps_per_s": round(1e6 / med, 1),
         "attention_layer_latency_us": r["step_us"],
         "wall_us_per_step": round(1e3 * r["ms_per_step"], 2),
         "algorithmic_bytes": kscan + gather,
         "whole_step_hbm_frac": round((kscan + gather) / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    if read_peak:
        e["whole_step_frac_of_measured_read_peak"] = round(
            (kscan + gather) / (med * 1e-6) / 1e9 / read_peak, 4)
    if r.get("graph_step_us"):
        e["graph_replay_step_us"] = r["graph_step_us"]
    ku = r.get("kernels_us")
    if ku and "score_pass1" in ku and "attend" in ku:
        ts_, ta = ku["score_pass1"] * 1e-6, ku["attend"] * 1e-6
        e["kernels_us"] = {kk: round(v, 2) for kk, v in ku.items()}
        e["kscan_frac"] = round(kscan / ts_ / 1e9 / HBM_PEAK_GBPS, 4)
        e["kscan_plus_gather_frac"] = round((kscan + gather) / (ts_ + ta) / 1e9 / HBM_PEAK_GBPS, 4)
    return e


def measure_configs(ts, W, steps, warmup, read_peak):
    """Decode steps (selection every step) at the other decode workloads: the
    tiny fp32 case, the Qwen2-7B shape at 32K tokens, the Llama-3-8B shape
    with 4 x 128K tokens. K/V copies rotate so that about 768 MB are touched
    between two uses of a copy (at least 3 copies)."""
    res = {}
    for name, cfg in (("tiny-4q2kv-d64-4k-f32", W.TINY),
                      ("qwen2-7b-shape-32k", W.QWEN_32K),
                      ("llama3-8b-shape-4x128k", W.LLAMA_4x128K)):
        kv = 2 * cfg.batch * cfg.seq_len * kv_bytes_per_token(cfg)
        copies = max(3, min(64, -(-768_000_000 // kv)))
        r, _ = measure_decode(ts, W, cfg, steps, warmup, copies, 1.0, True, name, graph=True)
        res[name] = config_entry(cfg, r, read_peak)
        res[name]["kv_copies"] = copies
    return res


def measure_read_peak(nbytes=1 << 30, reps=5):
    """The read bandwidth this machine reaches without any of this library's code:
    the best of a few torch reductions over 1 GiB of bf16 (a whole-tensor sum
    and row-wise sums and maxima over 8192- and 65536-element rows, fp32
    accumulation), each timed with HIP events, best of `reps`.
    Returns (GB/s, the op that reached it)."""
    import torch
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    ops = {
        "sum": lambda: x.sum(dtype=torch.float32),
        "rowsum8192": lambda: x.view(-1, 8192).sum(dim=1, dtype=torch.float32),
        "rowsum65536": lambda: x.view(-1, 65536).sum(dim=1, dtype=torch.float32),
        "rowmax8192": lambda: x.view(-1, 8192).amax(dim=1),
    }
    best, best_op = float("inf"), None
    for name, op in ops.items():
        for _ in range(2):
            op()
        torch.cuda.synchronize()
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            op()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            if t < best:
                best, best_op = t, name
    del x
    torch.cuda.empty_cache()
    return round(nbytes / best / 1e9, 1), best_op


def gpu_clock():
    """The GPU's reported current clocks (not pinned), or None."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
        card = d[sorted(d)[0]]
        pick = {k: v for k, v in card.items() if "sclk" in k.lower() or "mclk" in k.lower()}
        return pick or None
    except Exception:
        return None


def stored_fetch(path_name, key):
    """A counter figure (bytes) recorded in a profiles/ summary, or None."""
    try:
        with open(os.path.join(ROOT, "profiles", path_name)) as fh:
            for ln in fh:
                if ln.strip().startswith(key):
                    return int(ln.split(":", 1)[1].split()[0].replace(",", ""))
    except (OSError, ValueError, IndexError):
        return None
    return None


def cpu_single_thread(O, W, seconds=3.0):
    """The oracle with one BLAS thread on the tiny fp32 workload and the
    Qwen2-7B shape at 32K tokens: seconds per decode step (selection +
    sparse attention), on host copies generated from the same seeds."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return None
    out = {}
    with threadpool_limits(limits=1):
        for name, cfg in (("tiny-4q2kv-d64-4k-f32", W.TINY), ("qwen2-7b-shape-32k", W.QWEN_32K)):
            x = W.gen_decode(cfg, device="cpu")
            q = x["q"][0].float().double().numpy()
            K = x["k_cache"][0].float().numpy()
            V = x["v_cache"][0].float().numpy()
            n, t0 = 0, time.perf_counter()
            while True:
                S, _ = O.select(q, K, cfg.k)
                O.sparse_attention(q, K, V, S)
                n += 1
                el = time.perf_counter() - t0
                if el >= seconds or n >= 200:
                    break
            out[name] = {"s_per_step": round(el / n, 5), "steps": n, "threads": 1}
    return out


def cpu_baseline(O, W, cfg, x, seconds):
    """The fp64 oracle (as written, untuned) on host copies of the same inputs."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    q = x["q"][0].float().double().cpu().numpy()
    K = x["k_cache"][0].float().cpu().numpy()
    V = x["v_cache"][0].float().cpu().numpy()
    n = 0
    t0 = time.perf_counter()
    while True:
        S, _ = O.select(q, K, cfg.k)
        O.sparse_attention(q, K, V, S)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 50:
            break
    return {"value": n / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} full decode steps (selection + sparse attention, fp64 NumPy) of the "
                      f"same workload on host copies; {el:.1f} s; BLAS threads {threads} of "
                      f"{len(os.sched_getaffinity(0))} host cores"}


def profile_only(ts, W, name, steps, warmup):
    """One workload's steps alone, for kernel traces and hardware counters."""
    import torch
    if name == "prefill-512x64k":
        cfg = W.PREFILL_64K
        x = W.gen_prefill(cfg, device="cuda")
        q0 = x["q_pos0"]
        votes = torch.empty(cfg.chunk, cfg.n_ctx, dtype=torch.float32, device="cuda")
        idx = torch.empty(cfg.chunk, cfg.k, dtype=torch.int32, device="cuda")
        out = torch.empty(cfg.chunk, cfg.num_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
        ws = ts.Workspace()
        for i in range(warmup + steps):
            ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k, votes=votes, idx=idx)
            ts.sparse_attend_prefill(x["q"], x["k_cache"], x["v_cache"], q0, idx, out=out, ws=ws)
        torch.cuda.synchronize()
        print(json.dumps({"profile_only": name, "chunks": warmup + steps}), flush=True)
        return
    if name == "selcache-run":
        r = measure_selcache_run(ts, W)
        print(json.dumps({"profile_only": name, "us_per_step": r["us_per_step"]}), flush=True)
        return
    cfgs = {"qwen2-7b-shape-128k": (W.QWEN_128K, 6, 1.0), "qwen2-7b-shape-128k-hit": (W.QWEN_128K, 6, 0.9),
            "qwen2-7b-shape-32k": (W.QWEN_32K, 12, 1.0), "llama3-8b-shape-4x128k": (W.LLAMA_4x128K, 3, 1.0),
            "tiny-4q2kv-d64-4k-f32": (W.TINY, 64, 1.0)}
    cfg, copies, theta = cfgs[name]
    r, _ = measure_decode(ts, W, cfg, steps, warmup, copies, theta, False, name, nstat=1)
    print(json.dumps({"profile_only": name, "us_per_step": round(1e3 * r["ms_per_step"], 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--kv-copies", type=int, default=6)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--no-hit", action="store_true", help="skip the selection-reuse measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk measurement")
    ap.add_argument("--no-dense", action="store_true", help="skip the full-attention baseline")
    ap.add_argument("--no-loop", action="store_true", help="skip the multi-layer decode loop")
    ap.add_argument("--loop-layers", type=int, default=28)
    ap.add_argument("--no-quest", action="store_true", help="skip the page-selection variant")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 32K and 4x128K decode shapes and the 256-step selection-cache run")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB copy kernel (for HBM byte counters)")
    ap.add_argument("--profile-only", default=None,
                    choices=["qwen2-7b-shape-128k", "qwen2-7b-shape-128k-hit", "qwen2-7b-shape-32k",
                             "llama3-8b-shape-4x128k", "tiny-4q2kv-d64-4k-f32", "selcache-run",
                             "prefill-512x64k"],
                    help="only run --warmup then --steps steps of one workload (for rocprofv3 "
                         "kernel traces and counters); prints one short JSON line")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        _die_multi_gpu(max(args.gpus, world))

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    sys.path.insert(0, ROOT)
    import sparse_kv_cache_ts_amd as ts
    import workloads as W
    ts.load()
    if args.profile_only:
        profile_only(ts, W, args.profile_only, args.steps, args.warmup)
        return

    cfg = W.QWEN_128K
    read_peak, read_op = measure_read_peak()
    miss, x = measure_decode(ts, W, cfg, args.steps, args.warmup, args.kv_copies, 1.0,
                             not args.no_profile, "miss", graph=True)
    extra = {"gpu_clock": gpu_clock(), "measured_read_peak_GBps": read_peak,
             "measured_read_peak_op": f"torch {read_op} over 1 GiB of bf16 (best of several reductions)"}
    kscan_bytes, gather_bytes = decode_bytes(cfg)
    head = config_entry(cfg, miss, read_peak)
    head["graph_replay_step_us"] = miss.get("graph_step_us")
    head["eager_step_us"] = miss["step_us"]
    extra["headline_miss_step"] = head
    if not args.no_hit:
        hitres, _ = measure_decode(ts, W, cfg, args.steps, args.warmup, args.kv_copies, 0.9,
                                   not args.no_profile, "hit", graph=True)
        extra["hit_step"] = {"step_us": hitres["step_us"],
                             "graph_step_us": hitres.get("graph_step_us"),
                             "wall_us_per_step": round(1e3 * hitres["ms_per_step"], 2),
                             "gathered_bytes": gather_bytes,
                             "last_step_hits": hitres["last_step_hits"],
                             "kernels_us": {k: round(v, 2) for k, v in hitres.get("kernels_us", {}).items()}}

    roof = None
    if "kernels_us" in miss:
        ku = miss["kernels_us"]
        t_scan = ku["score_pass1"] * 1e-6
        t_att = ku["attend"] * 1e-6
        achieved = kscan_bytes / t_scan / 1e9
        kg = (kscan_bytes + gather_bytes) / (t_scan + t_att) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": stored_traffic(),
                "kernel": "score_pass1 (K-scan)", "bytes_per_launch": kscan_bytes,
                "avg_launch_us": round(ku["score_pass1"], 2),
                "frac_of_measured_read_peak": round(achieved / read_peak, 4) if read_peak else None,
                "kscan_plus_gather": {"bytes": kscan_bytes + gather_bytes, "GBps": round(kg, 1),
                                      "frac": round(kg / HBM_PEAK_GBPS, 4),
                                      "frac_of_measured_read_peak":
                                          round(kg / read_peak, 4) if read_peak else None}}
        extra["kernels_us"] = {kk: round(v, 2) for kk, v in ku.items()}
        extra["profiled_ms_per_step"] = round(miss["profiled_ms_per_step"], 4)
    extra["attention_layer_latency_us"] = miss["step_us"]
    extra["step_algorithmic_bytes"] = kscan_bytes + gather_bytes
    extra["whole_step_hbm_frac"] = round(
        (kscan_bytes + gather_bytes) / (miss["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)

    if not args.no_prefill:
        extra["prefill_chunk"] = measure_prefill(ts, W)
        past_l2 = stored_fetch("prefill_sparse_attention_512x4096_fetch.txt", "fetched_past_l2_bytes")
        if past_l2:
            att_us = extra["prefill_chunk"]["sparse_attention_us"]
            extra["prefill_chunk"]["sparse_attention_past_l2"] = {
                "bytes": past_l2, "GBps": round(past_l2 / (att_us * 1e-6) / 1e9, 1),
                "frac": round(past_l2 / (att_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    if not args.no_dense:
        dense = measure_dense(ts, W, cfg, args.steps, args.warmup, args.kv_copies)
        step_us = miss["step_us"]["median"]
        dense["speedup_vs_miss_step"] = round(dense["us_per_call"] / step_us, 3)
        if "hit_step" in extra:
            dense["speedup_vs_hit_step"] = round(dense["us_per_call"] / extra["hit_step"]["step_us"]["median"], 3)
        if "kernels_us" in miss:
            sparse_att = miss["kernels_us"]["attend"] + miss["kernels_us"]["combine"]
            dense["sparse_attention_us"] = round(sparse_att, 2)
            dense["attention_speedup"] = round(dense["us_per_call"] / sparse_att, 2)
        extra["dense_attention"] = dense

    if not args.no_loop:
        extra["decode_loop"] = measure_loop(ts, W, cfg, args.loop_layers,
                                            max(1, args.steps // 4), max(1, args.warmup // 4))

    if not args.no_quest:
        extra["quest_pages"] = measure_quest(ts, W, max(1, args.steps // 4), max(1, args.warmup // 4))

    if not args.no_configs:
        extra["other_decode_shapes"] = measure_configs(ts, W, max(1, args.steps // 2),
                                                       max(1, args.warmup // 2), read_peak)
        extra["selcache_run"] = measure_selcache_run(ts, W)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ts_oracle as O
        cpu = cpu_baseline(O, W, cfg, x, args.cpu_seconds)
        st = cpu_single_thread(O, W)
        if st:
            cpu["single_thread"] = st

    line = {
        "metric": "decode steps/sec + K-scan HBM GB/s (frac. of peak), Qwen2-7B shape, N=128K",
        "value": round(miss["steps_per_s"], 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(miss["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen2-7b-shape decode step, N=131072, batch 1, top-k 2048, "
                               "selection every step (theta=1.0)",
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "seq_len": cfg.seq_len, "batch": cfg.batch, "k": cfg.k,
                   "kv_dtype": "bf16", "accumulate": "f32", "kv_copies": args.kv_copies},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
