"""Parity at the full workload sizes, launched as bench.py launches them.

* Qwen2-7B attention shape (28/4 heads, d=128, bf16) at N=32768 and N=131072,
  batch 1, k=2048, 1% heavy keys: one decode step with theta = 1.0, so the
  whole path (cache check, K-scan, votes, top-k, sparse attention) runs.
* Llama-3-8B shape (32/8 heads), 4 sequences of 131072 tokens, k=4096, with
  heavy keys and with 16 planted keys.
* The tiny fp32 case (4/2 heads, d=64, 4096 tokens, 16 planted keys).
* The 256-step selection-cache run over 8 paged sequences of 16K..256K
  tokens (theta = 0.9): every decision, every miss step's selection and
  every step's output.

The oracle runs on exact host copies of the same inputs.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import ts_oracle as O
from tests.parity import check_attention, check_run, check_selection, np32, np64, oracle_votes

pytestmark = pytest.mark.gpu


def _decode_full(ts, cfg, planted_must=True):
    x = W.gen_decode(cfg, device="cuda")
    cache = ts.SelCache(cfg.batch, cfg.num_q_heads, cfg.head_dim, cfg.k)
    out, idx, hit = cache.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"], 1.0)
    torch.cuda.synchronize()
    cache.close()
    assert hit.sum().item() == 0
    lens = x["seq_lens"].tolist()
    gidx = idx.cpu().numpy()
    o = np64(out)
    q64 = np64(x["q"])
    tol = 1e-5 if cfg.dtype == "f32" else 1e-2
    for b in range(cfg.batch):
        n = lens[b]
        K = np32(x["k_cache"][b, :n])
        V = np32(x["v_cache"][b, :n])
        v_ref = oracle_votes(q64[b], K, n)
        assert abs(v_ref.sum() - cfg.num_q_heads) < 1e-9 * cfg.num_q_heads
        check_selection(gidx[b], v_ref, cfg.k)
        sp = x["special"][b].cpu().numpy()
        if planted_must and len(sp) <= cfg.k:
            assert set(sp.tolist()) <= set(gidx[b].tolist()), "a planted/heavy key was not selected"
        ref = O.sparse_attention(q64[b], K, V, gidx[b])
        check_attention(o[b], ref, tol)
        del K, V


@pytest.mark.parametrize("cfg", [W.TINY, W.QWEN_32K, W.QWEN_128K], ids=lambda c: c.name)
def test_decode_step_full_size(gpu_lib, cfg):
    _decode_full(gpu_lib, cfg)


def test_decode_step_llama_4x128k(gpu_lib):
    _decode_full(gpu_lib, W.LLAMA_4x128K)


def test_decode_step_llama_4x128k_planted(gpu_lib):
    from dataclasses import replace
    cfg = replace(W.LLAMA_4x128K, name="llama3-8b-shape-4x128k-planted16", heavy_frac=0.0,
                  planted=16)
    _decode_full(gpu_lib, cfg)


def test_score_votes_full_size(gpu_lib):
    """ts_score's vote row at N=131072 against the oracle, entry by entry."""
    ts = gpu_lib
    cfg = W.QWEN_128K
    x = W.gen_decode(cfg, device="cuda")
    votes = ts.score(x["q"], x["k_cache"], x["seq_lens"])
    torch.cuda.synchronize()
    n = cfg.seq_len
    ref = oracle_votes(np64(x["q"])[0], np32(x["k_cache"][0]), n)
    v = np64(votes[0, :n])
    err = np.abs(v - ref)
    assert (err <= 2e-4 * ref + 1e-7 * ref.max()).all()
    assert abs(v.sum() - cfg.num_q_heads) < 1e-4 * cfg.num_q_heads


@pytest.mark.timeout(1200)
def test_selection_cache_run_full_size(gpu_lib):
    """256 steps x 8 paged sequences: misses exactly at the jumps (t % 32 == 0);
    every decision, the selection of every miss step (8 per sequence) and the
    attention output of every step (2048 in all) against the oracle."""
    rc = W.SELCACHE_RUN
    hits = check_run(gpu_lib, rc, 0, rc.theta, sel_steps=None, att_steps=None)
    for t in range(rc.steps):
        assert (hits[t] == (0 if t % rc.jump_every == 0 else 1)).all(), f"step {t}"


def test_topk_rows_beyond_the_lds_bitmap(gpu_lib):
    """Rows longer than 262144 tokens: the selection bitmap lives in HBM, and
    ties/overflowing candidate lists fall back to rescanning the row."""
    ts = gpu_lib
    g = torch.Generator(device="cpu").manual_seed(77)
    lens = [262145, 300000, 600000, 431111]
    stride = 600000
    rows = [torch.rand(stride, generator=g),
            torch.randint(0, 4, (stride,), generator=g).float(),
            torch.exp(torch.randn(stride, generator=g) * 8),
            torch.randn(stride, generator=g)]
    votes = torch.stack(rows)
    for k in (1, 4096, 20000):
        idx = ts.topk(votes.cuda(), torch.tensor(lens, dtype=torch.int32, device="cuda"), k)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        v = votes.numpy().astype(np.float64)
        for r, n in enumerate(lens):
            assert np.array_equal(got[r], O.top_k(v[r, :n], k)), f"row {r} (len {n}), k {k}"


def test_decode_step_300k_tokens(gpu_lib):
    """One sequence of 300000 tokens (beyond the LDS bitmap), 8/2 heads."""
    cfg = W.DecodeConfig("g4-d128-bf16-300k", batch=1, num_q_heads=8, num_kv_heads=2,
                         head_dim=128, seq_len=300000, dtype="bf16", k=4096, seed=78,
                         heavy_frac=0.01)
    _decode_full(gpu_lib, cfg)


@pytest.mark.parametrize("cfg", [
    W.DecodeConfig("g8-d64-bf16-131k", batch=2, num_q_heads=32, num_kv_heads=4, head_dim=64,
                   seq_len=131072, dtype="bf16", k=2048, seed=79, heavy_frac=0.01),
    W.DecodeConfig("g4-d128-f32-65k", batch=1, num_q_heads=16, num_kv_heads=4, head_dim=128,
                   seq_len=65536, dtype="f32", k=1024, seed=80, heavy_frac=0.01),
], ids=lambda c: c.name)
def test_decode_step_other_full_sizes(gpu_lib, cfg):
    """head_dim 64 on the matrix-core attention (2 k-steps, one 16-dimension
    tile per wave) and fp32 rows (the row-group attention), both with the
    selection finished inside the attention work-groups."""
    _decode_full(gpu_lib, cfg)
