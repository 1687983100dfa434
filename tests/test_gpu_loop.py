"""The decode loop on a growing cache: ts_append_kv, then ts_decode_step, per token.

* Append is byte work: the cache after appends must equal, byte for byte, the
  same rows written by indexing on the host; lengths advance by one; a position
  at the capacity is skipped and its length kept.
* A loop of append + decode steps is checked against the oracle's selection
  cache run over the grown prefix (decisions, selections, attention), with the
  parity rules of tests/parity.py.
* The same loop captured once as a HIP graph and replayed for every token must
  reproduce the eager loop bit for bit, replay after replay, with eager work and
  synchronisations between the replays.
"""
import math
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import check_attention, check_selection, np32, np64, oracle_votes

pytestmark = pytest.mark.gpu


def _host_pos(page_table, b, pos, P):
    if page_table is None:
        return (b, pos)
    return (int(page_table[b, pos // P]), pos % P)


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_kv_places_rows(gpu_lib, paged, dtype):
    ts = gpu_lib
    cfg = replace(W.LOOP_RUN, dtype=dtype, steps=5, min_len=1, max_len=300)
    x = W.gen_loop(cfg, paged, device="cuda")
    kc, vc, pt = x["k_cache"], x["v_cache"], x["page_table"]
    lens = x["seq_lens"].clone()
    ref_k, ref_v = kc.cpu().clone(), vc.cpu().clone()
    pt_h = None if pt is None else pt.cpu()
    lens_h = lens.cpu().tolist()
    for t in range(cfg.steps):
        ts.append_kv(x["k_new"][t], x["v_new"][t], kc, vc, lens, page_table=pt)
        for b in range(cfg.batch):
            at = _host_pos(pt_h, b, lens_h[b], cfg.page_size)
            ref_k[at] = x["k_new"][t, b].cpu()
            ref_v[at] = x["v_new"][t, b].cpu()
            lens_h[b] += 1
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == lens_h
    assert torch.equal(kc.cpu().view(torch.uint8), ref_k.view(torch.uint8))
    assert torch.equal(vc.cpu().view(torch.uint8), ref_v.view(torch.uint8))


def test_append_kv_skips_full_sequence(gpu_lib):
    """A sequence already at max_len keeps its length and its cache unchanged."""
    ts = gpu_lib
    cfg = replace(W.LOOP_RUN, steps=1, batch=2, min_len=10, max_len=10)
    x = W.gen_loop(cfg, False, device="cuda")
    kc, vc = x["k_cache"], x["v_cache"]           # capacity 11
    lens = torch.tensor([11, 10], dtype=torch.int32, device="cuda")
    before = kc.clone()
    ts.append_kv(x["k_new"][0], x["v_new"][0], kc, vc, lens)
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == [11, 11]
    assert torch.equal(kc[0], before[0])
    assert torch.equal(kc[1, 10], x["k_new"][0, 1])
    assert torch.equal(vc[1, 10], x["v_new"][0, 1])


def _grown(x, cfg, lens0, paged):
    """Host fp32 K, V of each sequence after all appends: [B] arrays [len0+T][Hkv][d]."""
    kc, vc, pt = np32(x["k_cache"]), np32(x["v_cache"]), x["page_table"]
    kn, vn = np32(x["k_new"]), np32(x["v_new"])
    Ks, Vs = [], []
    for b in range(cfg.batch):
        n = lens0[b]
        if paged:
            from oracle import ts_oracle as O
            ptb = pt[b].cpu().numpy()
            K0, V0 = O.paged_to_contiguous(kc, ptb, n), O.paged_to_contiguous(vc, ptb, n)
        else:
            K0, V0 = kc[b, :n], vc[b, :n]
        Ks.append(np.concatenate([K0, kn[:, b]]))
        Vs.append(np.concatenate([V0, vn[:, b]]))
    return Ks, Vs


def _run_eager(ts, x, cfg, mode, theta):
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    lens = x["seq_lens"].clone()
    cache = ts.SelCache(cfg.batch, cfg.num_q_heads, cfg.head_dim, cfg.k, mode=mode)
    outs, sels, hits = [], [], []
    for t in range(cfg.steps):
        ts.append_kv(x["k_new"][t], x["v_new"][t], kc, vc, lens, page_table=x["page_table"])
        o, i, h = cache.decode_step(x["queries"][t], kc, vc, lens, theta,
                                    page_table=x["page_table"])
        outs.append(o.clone())
        sels.append(i.clone())
        hits.append(h.clone())
    torch.cuda.synchronize()
    cache.close()
    return torch.stack(outs), torch.stack(sels), torch.stack(hits), lens


@pytest.mark.parametrize("paged,mode", [(False, 0), (True, 1)], ids=["contiguous-m0", "paged-m1"])
def test_decode_loop_vs_oracle(gpu_lib, paged, mode):
    from oracle import ts_oracle as O
    ts = gpu_lib
    cfg = W.LOOP_RUN
    theta = cfg.theta
    x = W.gen_loop(cfg, paged, device="cuda")
    lens0 = x["seq_lens"].tolist()
    outs, sels, hits, lens = _run_eager(ts, x, cfg, mode, theta)
    assert lens.cpu().tolist() == [n + cfg.steps for n in lens0]
    outs, sels, hits = np64(outs), sels.cpu().numpy(), hits.cpu().numpy()
    assert 0 < hits.sum() < hits.size, "the run should mix hits and misses"
    Q = np64(x["queries"])
    Ks, Vs = _grown(x, cfg, lens0, paged)
    for b in range(cfg.batch):
        ref_cache = O.SelectionCache(mode)
        for t in range(cfg.steps):
            n = lens0[b] + t + 1
            hit_ref, c = ref_cache.decide(Q[t, b], theta)
            if abs(c - theta) > 1e-9 or math.isnan(c):
                assert bool(hits[t, b]) == hit_ref, f"seq {b} step {t}: cos {c}"
            if hits[t, b]:
                assert np.array_equal(sels[t, b], sels[t - 1, b])
                # a reused selection never names the tokens appended since
                assert sels[t, b].max() < n - 1 or (sels[t, b] == -1).all()
            else:
                check_selection(sels[t, b], oracle_votes(Q[t, b], Ks[b], n), cfg.k)
            check_attention(outs[t, b], O.sparse_attention(Q[t, b], Ks[b][:n], Vs[b][:n],
                                                           sels[t, b]), 1e-2)
            if mode == 0 or not hits[t, b]:
                ref_cache.prev_q = Q[t, b].copy()
            ref_cache.prev_S = sels[t, b]
            ref_cache.valid = True


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_decode_loop_graph_replay(gpu_lib, paged):
    """append + decode_step captured once, replayed per token == the eager loop."""
    ts = gpu_lib
    cfg = W.LOOP_RUN
    x = W.gen_loop(cfg, paged, device="cuda")
    e_out, e_idx, e_hit, e_lens = _run_eager(ts, x, cfg, 0, cfg.theta)

    kc, vc, pt = x["k_cache"].clone(), x["v_cache"].clone(), x["page_table"]
    lens = x["seq_lens"].clone()
    B, Hq, d = cfg.batch, cfg.num_q_heads, cfg.head_dim
    cache = ts.SelCache(B, Hq, d, cfg.k, mode=0)
    q_in = torch.empty_like(x["queries"][0])
    kn_in, vn_in = torch.empty_like(x["k_new"][0]), torch.empty_like(x["v_new"][0])
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, cfg.k, dtype=torch.int32, device="cuda")
    hit = torch.empty(B, dtype=torch.int32, device="cuda")
    L = ts.make_layout(q_in, kc, pt)
    cache.ws.get(cache.workspace_size(L, B), q_in.device)     # no allocation while capturing
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ts.append_kv(kn_in, vn_in, kc, vc, lens, page_table=pt)
        cache.decode_step(q_in, kc, vc, lens, cfg.theta, page_table=pt, out=out, idx_out=idx,
                          hit_out=hit)
    # capturing runs nothing: the state is untouched until the first replay
    assert torch.equal(lens, x["seq_lens"])
    for t in range(cfg.steps):
        q_in.copy_(x["queries"][t])
        kn_in.copy_(x["k_new"][t])
        vn_in.copy_(x["v_new"][t])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(hit, e_hit[t]), f"step {t}"
        assert torch.equal(idx, e_idx[t]), f"step {t}"
        assert torch.equal(out, e_out[t]), f"step {t}"
    assert torch.equal(lens, e_lens)
    h, m = cache.stats(B)
    assert h == e_hit.sum(0).tolist()
    cache.close()


def test_decode_loop_layers_graph(gpu_lib):
    """Three layers, each with its own cache, lengths and selection-cache state:
    one graph holding every layer's append + decode step, replayed per token,
    equals each layer run alone eagerly (state stays per layer)."""
    ts = gpu_lib
    cfgs = [replace(W.LOOP_RUN, seed=W.LOOP_RUN.seed + 10 * l, steps=10) for l in range(3)]
    xs = [W.gen_loop(c, True, device="cuda") for c in cfgs]
    alone = [_run_eager(ts, x, c, 0, c.theta) for x, c in zip(xs, cfgs)]
    B, Hq, d, k = cfgs[0].batch, cfgs[0].num_q_heads, cfgs[0].head_dim, cfgs[0].k
    lay = []
    for x in xs:
        st = {"k": x["k_cache"].clone(), "v": x["v_cache"].clone(), "lens": x["seq_lens"].clone(),
              "pt": x["page_table"], "cache": ts.SelCache(B, Hq, d, k, mode=0),
              "q": torch.empty_like(x["queries"][0]), "kn": torch.empty_like(x["k_new"][0]),
              "vn": torch.empty_like(x["v_new"][0]),
              "out": torch.empty(B, Hq, d, dtype=torch.float32, device="cuda"),
              "idx": torch.empty(B, k, dtype=torch.int32, device="cuda"),
              "hit": torch.empty(B, dtype=torch.int32, device="cuda")}
        L = ts.make_layout(st["q"], st["k"], st["pt"])
        st["cache"].ws.get(st["cache"].workspace_size(L, B), st["q"].device)
        lay.append(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for st in lay:
            ts.append_kv(st["kn"], st["vn"], st["k"], st["v"], st["lens"], page_table=st["pt"])
            st["cache"].decode_step(st["q"], st["k"], st["v"], st["lens"], cfgs[0].theta,
                                    page_table=st["pt"], out=st["out"], idx_out=st["idx"],
                                    hit_out=st["hit"])
    for t in range(cfgs[0].steps):
        for st, x in zip(lay, xs):
            st["q"].copy_(x["queries"][t])
            st["kn"].copy_(x["k_new"][t])
            st["vn"].copy_(x["v_new"][t])
        graph.replay()
        torch.cuda.synchronize()
        for l, st in enumerate(lay):
            e_out, e_idx, e_hit, _ = alone[l]
            assert torch.equal(st["hit"], e_hit[t]), f"layer {l} step {t}"
            assert torch.equal(st["idx"], e_idx[t]), f"layer {l} step {t}"
            assert torch.equal(st["out"], e_out[t]), f"layer {l} step {t}"
    for l, st in enumerate(lay):
        assert torch.equal(st["lens"], alone[l][3])
        st["cache"].close()
