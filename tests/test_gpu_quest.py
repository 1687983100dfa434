"""GPU parity of Quest-style page selection against oracle/quest_oracle.py.

* Page extremes are byte work on stored values: bit-exact (compared as values).
* Page scores: fp32 against fp64, |s - s_ref| <= SCORE_TOL * mag per row, with
  mag = scale * max over pages of sum_c max_h |q_hc| * max(|min_c|, |max_c|),
  the size of the terms the fp32 sums add.
* Page selection: exact count, ascending, -1 padded; every page whose oracle
  score lies more than 2 * SCORE_TOL * mag from the k-th score is inside or
  outside the selection exactly as in the oracle's.
* Attention: the oracle's page attention over the GPU's own pages, per head
  max error <= 1e-2 * max |ref| (as for token selection).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import check_attention, np32, np64

pytestmark = pytest.mark.gpu

SCORE_TOL = 4e-6

SMALL = [
    W.RunConfig("quest-3seq-16x4-d128-p16", steps=1, batch=3, num_q_heads=16, num_kv_heads=4,
                head_dim=128, min_len=1, max_len=3000, dtype="bf16", k=512, seed=71),
    W.RunConfig("quest-2seq-8x8-d64-p32-f32", steps=1, batch=2, num_q_heads=8, num_kv_heads=8,
                head_dim=64, min_len=500, max_len=2000, dtype="f32", k=256, seed=72, page_size=32),
    W.RunConfig("quest-2seq-28x4-d128-p16", steps=1, batch=2, num_q_heads=28, num_kv_heads=4,
                head_dim=128, min_len=2000, max_len=5000, dtype="bf16", k=1024, seed=73),
    W.RunConfig("quest-2seq-32x4-d64-p4", steps=1, batch=2, num_q_heads=32, num_kv_heads=4,
                head_dim=64, min_len=100, max_len=900, dtype="bf16", k=64, seed=74, page_size=4),
    # 3, 5 and 6 query heads per KV head
    W.RunConfig("quest-2seq-6x2-d128-p16", steps=1, batch=2, num_q_heads=6, num_kv_heads=2,
                head_dim=128, min_len=800, max_len=2500, dtype="bf16", k=256, seed=75),
    W.RunConfig("quest-1seq-20x4-d64-p16-f32", steps=1, batch=1, num_q_heads=20, num_kv_heads=4,
                head_dim=64, min_len=1500, max_len=1500, dtype="f32", k=320, seed=76),
    W.RunConfig("quest-2seq-24x4-d128-p32", steps=1, batch=2, num_q_heads=24, num_kv_heads=4,
                head_dim=128, min_len=1000, max_len=4000, dtype="bf16", k=512, seed=77, page_size=32),
]


def _seq(x, b, n):
    from oracle import ts_oracle as O
    pt = x["page_table"][b].cpu().numpy()
    return (O.paged_to_contiguous(np32(x["k_pool"]).astype(np.float64), pt, n),
            O.paged_to_contiguous(np32(x["v_pool"]).astype(np.float64), pt, n))


def _mag(q, kmin, kmax, G, scale):
    Hq, d = q.shape
    Hkv = kmin.shape[1]
    qa = np.abs(q).reshape(Hkv, G, d).max(axis=1)                 # [Hkv][d]
    ext = np.maximum(np.abs(kmin), np.abs(kmax))                  # [pages][Hkv][d]
    return scale * (ext * qa[None]).sum(axis=2).max(axis=0)       # [Hkv]


def _check_pages(sel, s_ref, k_pages, band):
    n = s_ref.shape[0]
    k_eff = min(k_pages, n)
    assert (sel[k_eff:] == -1).all(), "padding must be -1"
    s = sel[:k_eff]
    assert (s >= 0).all() and (s < n).all() and (np.diff(s) > 0).all()
    if k_eff == 0:
        return
    order = np.lexsort((np.arange(n), -s_ref))
    sk = s_ref[order[k_eff - 1]]
    decided = np.abs(s_ref - sk) > band
    want = np.zeros(n, bool)
    want[order[:k_eff]] = True
    got = np.zeros(n, bool)
    got[s] = True
    bad = decided & (want != got)
    assert not bad.any(), f"{bad.sum()} decided pages differ"


def _run(ts, x, cfg, q):
    lens = x["seq_lens"]
    meta = ts.quest_meta(x["k_pool"], x["page_table"], lens)
    k_pages = max(1, cfg.k // cfg.page_size)
    n_pages = x["page_table"].shape[1]
    scores = torch.zeros(cfg.batch, cfg.num_kv_heads, n_pages, dtype=torch.float32, device="cuda")
    pidx, scores = ts.quest_select(q, x["k_pool"], meta, x["page_table"], lens, k_pages,
                                   scores=scores)
    out = ts.quest_attend(q, x["k_pool"], x["v_pool"], x["page_table"], lens, pidx)
    torch.cuda.synchronize()
    return meta, pidx, scores, out, k_pages


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_quest_meta_select_attend(gpu_lib, cfg):
    from oracle import quest_oracle as Q
    ts = gpu_lib
    x = W.gen_run(cfg, device="cuda")
    q = x["queries"][0]
    meta, pidx, scores, out, k_pages = _run(ts, x, cfg, q)
    lens = x["seq_lens"].tolist()
    Qh, meta_h, pt = np64(q), np32(meta), x["page_table"].cpu().numpy()
    pidx, scores, out = pidx.cpu().numpy(), np64(scores), np64(out)
    G = cfg.num_q_heads // cfg.num_kv_heads
    scale = 1.0 / np.sqrt(cfg.head_dim)
    P = cfg.page_size
    for b, n in enumerate(lens):
        K, V = _seq(x, b, n)
        kmin, kmax = Q.page_extremes(K, P)
        n_pages = kmin.shape[0]
        # extremes: exact, stored at the pool page of each logical page
        assert np.array_equal(meta_h[pt[b, :n_pages], :, 0], kmin)
        assert np.array_equal(meta_h[pt[b, :n_pages], :, 1], kmax)
        s_ref = Q.page_scores(Qh[b], kmin, kmax)
        mag = _mag(Qh[b], kmin, kmax, G, scale)
        for g in range(cfg.num_kv_heads):
            err = np.abs(scores[b, g, :n_pages] - s_ref[g]).max()
            assert err <= SCORE_TOL * mag[g], (b, g, err, mag[g])
            _check_pages(pidx[b, g], s_ref[g], k_pages, 2 * SCORE_TOL * mag[g])
        ref = Q.page_attention(Qh[b], K, V, pidx[b], P)
        check_attention(out[b], ref, 1e-2)


def test_quest_heavy_pages_selected(gpu_lib):
    """The workload's heavy keys point along step 0's first query head of each
    group: their pages top the scores of every KV head."""
    ts = gpu_lib
    cfg = replace(SMALL[0], min_len=2000, heavy_frac=0.002)
    x = W.gen_run(cfg, device="cuda")
    _, pidx, _, _, _ = _run(ts, x, cfg, x["queries"][0])
    pidx = pidx.cpu().numpy()
    for b, pos in enumerate(x["special"]):
        pages = set((pos.cpu().numpy() // cfg.page_size).tolist())
        for g in range(cfg.num_kv_heads):
            assert pages <= set(pidx[b, g].tolist())


def test_quest_edge_cases(gpu_lib):
    """Empty sequence, one partial page, k_pages beyond the pages, negative page entries."""
    from oracle import quest_oracle as Q
    ts = gpu_lib
    cfg = replace(SMALL[0], batch=3)
    x = W.gen_run(cfg, device="cuda", lens=[0, 5, 40])
    q = x["queries"][0]
    lens = x["seq_lens"]
    meta = ts.quest_meta(x["k_pool"], x["page_table"], lens)
    pidx, _ = ts.quest_select(q, x["k_pool"], meta, x["page_table"], lens, 4)
    torch.cuda.synchronize()
    p = pidx.cpu().numpy()
    assert (p[0] == -1).all()
    assert (p[1] == [[0, -1, -1, -1]] * 4).all()
    assert (p[2] == [[0, 1, 2, -1]] * 4).all()
    pidx2 = pidx.clone()
    pidx2[2, :, 1] = -1                                   # drop page 1 of sequence 2
    out = ts.quest_attend(q, x["k_pool"], x["v_pool"], x["page_table"], lens, pidx2)
    torch.cuda.synchronize()
    o = np64(out)
    assert (o[0] == 0).all()
    Qh = np64(q)
    for b in (1, 2):
        K, V = _seq(x, b, lens[b].item())
        check_attention(o[b], Q.page_attention(Qh[b], K, V, pidx2[b].cpu().numpy(),
                                               cfg.page_size), 1e-2)


def test_quest_meta_last_page_after_append(gpu_lib):
    """Append then refresh only the last page: equals a full rebuild, every step."""
    ts = gpu_lib
    cfg = replace(W.LOOP_RUN, steps=20, min_len=30, max_len=70)
    x = W.gen_loop(cfg, True, device="cuda")
    kc, vc, pt, lens = x["k_cache"], x["v_cache"], x["page_table"], x["seq_lens"].clone()
    meta = ts.quest_meta(kc, pt, lens)
    for t in range(cfg.steps):
        ts.append_kv(x["k_new"][t], x["v_new"][t], kc, vc, lens, page_table=pt)
        ts.quest_meta(kc, pt, lens, meta=meta, last_page_only=True)
        full = ts.quest_meta(kc, pt, lens)
        torch.cuda.synchronize()
        n_used = int(((lens.cpu() + cfg.page_size - 1) // cfg.page_size).sum())
        used = pt.cpu().numpy()
        used = np.concatenate([used[b, :(int(lens[b]) + cfg.page_size - 1) // cfg.page_size]
                               for b in range(cfg.batch)])
        assert used.size == n_used
        assert torch.equal(meta[used], full[used]), f"step {t}"


def test_quest_full_size(gpu_lib):
    """8 sequences of 16K..256K tokens, 32/8 heads, page 16, 256 pages per KV head:
    every row's scores and selection, and every sequence's attention."""
    from oracle import quest_oracle as Q
    ts = gpu_lib
    cfg = W.SELCACHE_RUN
    x = W.gen_run(cfg, device="cuda")
    q = x["queries"][0]
    meta, pidx, scores, out, k_pages = _run(ts, x, cfg, q)
    assert k_pages == 256
    lens = x["seq_lens"].tolist()
    Qh, pt = np64(q), x["page_table"].cpu().numpy()
    meta_h = np32(meta)
    pidx, scores, out = pidx.cpu().numpy(), np64(scores), np64(out)
    G = cfg.num_q_heads // cfg.num_kv_heads
    scale = 1.0 / np.sqrt(cfg.head_dim)
    kp = np32(x["k_pool"])
    vp = np32(x["v_pool"])
    del x
    for b, n in enumerate(lens):
        from oracle import ts_oracle as O
        K = O.paged_to_contiguous(kp, pt[b], n).astype(np.float64)
        kmin, kmax = Q.page_extremes(K, cfg.page_size)
        n_pages = kmin.shape[0]
        assert np.array_equal(meta_h[pt[b, :n_pages], :, 0], kmin)
        assert np.array_equal(meta_h[pt[b, :n_pages], :, 1], kmax)
        s_ref = Q.page_scores(Qh[b], kmin, kmax)
        mag = _mag(Qh[b], kmin, kmax, G, scale)
        for g in range(cfg.num_kv_heads):
            assert np.abs(scores[b, g, :n_pages] - s_ref[g]).max() <= SCORE_TOL * mag[g]
            _check_pages(pidx[b, g], s_ref[g], k_pages, 2 * SCORE_TOL * mag[g])
        V = O.paged_to_contiguous(vp, pt[b], n).astype(np.float64)
        ref = Q.page_attention(Qh[b], K, V, pidx[b], cfg.page_size)
        del K, V
        check_attention(out[b], ref, 1e-2)
