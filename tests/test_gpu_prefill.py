"""GPU parity of the chunked-prefill scoring (bf16 MFMA) against the fp64 oracle.

Votes: every visible entry within VOTE_RTOL * ref + VOTE_ATOL_REL_MAX * max(ref)
of the oracle's row on the same bf16 inputs, entries past the causal limit
exactly 0, every row summing to Hq. Selection: the decided-token rule of
tests/parity.py per row, with row i choosing from its own q_pos0 + i + 1 keys.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import ts_oracle as O
from tests.parity import check_selection, np32, np64

pytestmark = pytest.mark.gpu

VOTE_RTOL = 2e-4
VOTE_ATOL_REL_MAX = 1e-7


def _cfg(name, C, n_ctx, Hq, Hkv, d, k, seed, q_pos0=None):
    c = W.PrefillConfig(name, chunk=C, n_ctx=n_ctx, num_q_heads=Hq, num_kv_heads=Hkv,
                        head_dim=d, dtype="bf16", k=k, seed=seed)
    return c, (c.q_pos0 if q_pos0 is None else q_pos0)


SMALL = [
    _cfg("c100-n3000-h8x2-d128", 100, 3000, 8, 2, 128, 256, 31),
    _cfg("c64-n1000-h32x8-d64-mid", 64, 1000, 32, 8, 64, 128, 32, q_pos0=500),
    _cfg("c1-n777-h4x1-d128", 1, 777, 4, 1, 128, 700, 33),
    _cfg("c70-first-chunk-h16x4-d128", 70, 70, 16, 4, 128, 32, 34, q_pos0=0),
    _cfg("c257-n4099-h28x7-d128", 257, 4099, 28, 7, 128, 1000, 35),
    # query-head groups other than 4: padded to 1, 2, 4 or 8 slots per KV head
    _cfg("g1-c97-n2000-h8x8-d128", 97, 2000, 8, 8, 128, 300, 36),
    _cfg("g2-c130-n3333-h8x4-d64-mid", 130, 3333, 8, 4, 64, 500, 37, q_pos0=1500),
    _cfg("g3-c70-n1500-h6x2-d128", 70, 1500, 6, 2, 128, 200, 38),
    _cfg("g7-c129-n5000-h28x4-d128", 129, 5000, 28, 4, 128, 1024, 39),
    _cfg("g8-c64-n2500-h32x4-d64", 64, 2500, 32, 4, 64, 256, 40),
    _cfg("g5-c33-n900-h10x2-d128", 33, 900, 10, 2, 128, 100, 41),
]


# Chunks whose vote pass has more (query block, 512-key split) items than
# work-groups that run at once, so each vote work-group walks several
# consecutive splits: 3, 3 and 2 of them here, with a shorter last group
# (1, 2 and 1 splits), a partial last split (64, 305 and 124 keys), and for
# the mid-context chunk whole splits past every row's causal limit.
MULTI_SPLIT = [
    _cfg("c256-n40000-h32x8-d128", 256, 40000, 32, 8, 128, 2048, 42),
    _cfg("g7-c200-n30001-h28x4-d128-mid", 200, 30001, 28, 4, 128, 1024, 43, q_pos0=20000),
    _cfg("g2-c150-n50300-h16x8-d64", 150, 50300, 16, 8, 64, 1000, 44),
]


def _check_votes(votes_row, ref, n_vis, Hq):
    v = np64(votes_row)
    assert (v[n_vis:] == 0).all(), "votes past the causal limit must be 0"
    v = v[:n_vis]
    assert abs(v.sum() - Hq) < 1e-4 * Hq
    err = np.abs(v - ref)
    bound = VOTE_RTOL * ref + VOTE_ATOL_REL_MAX * ref.max()
    assert (err <= bound).all(), f"max rel err {(err / np.maximum(ref, 1e-30)).max():.3e}"


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0].name)
def test_prefill_votes_and_select(gpu_lib, case):
    """A chunk in the middle of the context leaves later keys unseen (all 0)."""
    ts = gpu_lib
    cfg, q0 = case
    x = W.gen_prefill(cfg, device="cuda")
    votes, idx = ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k)
    torch.cuda.synchronize()
    Q, K = np64(x["q"]), np32(x["k_cache"])
    refs = O.prefill_votes(Q, K, q0)
    gi = idx.cpu().numpy()
    for i, ref in enumerate(refs):
        _check_votes(votes[i], ref, q0 + i + 1, cfg.num_q_heads)
        # selection from the GPU's own vote row must be exact top-k of it ...
        assert (gi[i] == O.top_k(np32(votes[i, :q0 + i + 1]).astype(np.float64), cfg.k)).all()
        # ... and agree with the oracle's selection on every decided token
        check_selection(gi[i], ref, cfg.k)


@pytest.mark.parametrize("case", MULTI_SPLIT, ids=lambda c: c[0].name)
def test_prefill_multi_split_work_groups(gpu_lib, case):
    """Every row of the chunk: votes entry by entry against the oracle, zeros
    past the causal limit, and the selection (exact top-k of the GPU's own
    row, decided tokens as in the oracle's)."""
    ts = gpu_lib
    cfg, q0 = case
    x = W.gen_prefill(cfg, device="cuda")
    votes, idx = ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k)
    torch.cuda.synchronize()
    V32 = np32(votes)
    assert (V32[:, q0 + cfg.chunk:] == 0).all()
    gi = idx.cpu().numpy()
    refs = O.prefill_votes(np64(x["q"]), np64(x["k_cache"]), q0)
    for i, ref in enumerate(refs):
        n = q0 + i + 1
        _check_votes(votes[i], ref, n, cfg.num_q_heads)
        assert np.array_equal(gi[i], O.top_k(V32[i, :n].astype(np.float64), cfg.k)), f"row {i}"
        check_selection(gi[i], ref, cfg.k)


def test_prefill_score_matches_select_votes(gpu_lib):
    ts = gpu_lib
    cfg = SMALL[0][0]
    x = W.gen_prefill(cfg, device="cuda")
    v1 = ts.score_prefill(x["q"], x["k_cache"], x["q_pos0"])
    v2, _ = ts.select_prefill(x["q"], x["k_cache"], x["q_pos0"], cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(v1, v2)


@pytest.mark.timeout(900)
def test_prefill_full_size(gpu_lib):
    """512 queries over 65536 keys, 32/8 heads, d=128, in the launch bench.py
    times. Every row: zeros past its causal limit, a sum of Hq, and a
    selection equal to the exact top-k (oracle rule) of the GPU's own vote
    row. 64 rows spread over the chunk, the first and last included: votes
    entry by entry and the decided-token rule against the oracle."""
    ts = gpu_lib
    cfg = W.PREFILL_64K
    x = W.gen_prefill(cfg, device="cuda")
    q0 = x["q_pos0"]
    votes, idx = ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k)
    torch.cuda.synchronize()
    sums = votes.double().sum(dim=1)
    assert torch.allclose(sums, torch.full_like(sums, cfg.num_q_heads), rtol=1e-4)
    V32 = np32(votes)
    gi = idx.cpu().numpy()
    for r in range(cfg.chunk):
        n = q0 + r + 1
        assert (V32[r, n:] == 0).all(), f"row {r}: votes past the causal limit"
        assert np.array_equal(gi[r], O.top_k(V32[r, :n].astype(np.float64), cfg.k)), f"row {r}"
    rows = sorted(set(np.linspace(0, cfg.chunk - 1, 64).round().astype(int).tolist()))
    assert rows[0] == 0 and rows[-1] == cfg.chunk - 1 and len(rows) == 64
    Q, K = np64(x["q"]), np64(x["k_cache"])
    refs = O.prefill_votes(Q, K, q0, rows=rows)
    for r, ref in zip(rows, refs):
        _check_votes(votes[r], ref, q0 + r + 1, cfg.num_q_heads)
        check_selection(gi[r], ref, cfg.k)


def test_prefill_rejects_unsupported(gpu_lib):
    ts = gpu_lib
    q = torch.zeros(4, 32, 128, dtype=torch.bfloat16, device="cuda")   # G = 16
    k = torch.zeros(100, 2, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ts.TsError) as e:
        ts.score_prefill(q, k, 96)
    assert e.value.status == ts.TS_ERR_UNSUPPORTED
    q = torch.zeros(4, 8, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ts.TsError) as e:
        ts.score_prefill(q, k, 97)                                    # 97 + 4 > 100
    assert e.value.status == ts.TS_ERR_INVALID_ARG
    with pytest.raises(ts.TsError) as e:
        ts.score_prefill(q.float(), k.float(), 96)                    # fp32
    assert e.value.status == ts.TS_ERR_UNSUPPORTED


# G = 4 in several shapes, then 1, 7 (the Qwen2-7B layout) and 8 query heads
# per KV head, whose head slices the attention kernel lays out differently
ATT_CASES = [SMALL[0], SMALL[1], SMALL[3], SMALL[4], SMALL[5], SMALL[8], SMALL[9]]


@pytest.mark.parametrize("case", ATT_CASES, ids=lambda c: c[0].name)
def test_prefill_sparse_attention(gpu_lib, case):
    """Each query attends over its own selection (from select_prefill)."""
    from tests.parity import check_attention
    ts = gpu_lib
    cfg, q0 = case
    x = W.gen_prefill(cfg, device="cuda")
    _, idx = ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k)
    out = ts.sparse_attend_prefill(x["q"], x["k_cache"], x["v_cache"], q0, idx)
    torch.cuda.synchronize()
    Q, K, V = np64(x["q"]), np32(x["k_cache"]), np32(x["v_cache"])
    gi, o = idx.cpu().numpy(), np64(out)
    for i in range(cfg.chunk):
        n = q0 + i + 1
        ref = O.sparse_attention(Q[i], K[:n], V[:n], gi[i])
        check_attention(o[i], ref, 1e-2)


def test_prefill_sparse_attention_skips_invalid(gpu_lib):
    """Indices at or past a row's causal limit, and negative ones, are skipped."""
    from tests.parity import check_attention
    ts = gpu_lib
    cfg, q0 = SMALL[1]
    x = W.gen_prefill(cfg, device="cuda")
    C = cfg.chunk
    g = torch.Generator(device="cpu").manual_seed(5)
    idx = torch.randint(-3, cfg.n_ctx + 5, (C, 50), generator=g, dtype=torch.int32)
    idx[0, :] = -1                                   # a row with nothing valid
    out = ts.sparse_attend_prefill(x["q"], x["k_cache"], x["v_cache"], q0, idx.cuda())
    torch.cuda.synchronize()
    Q, K, V = np64(x["q"]), np32(x["k_cache"]), np32(x["v_cache"])
    gi, o = idx.numpy(), np64(out)
    assert (o[0] == 0).all()
    for i in range(1, C):
        n = q0 + i + 1
        sel = gi[i][(gi[i] >= 0) & (gi[i] < n)]
        ref = O.sparse_attention(Q[i], K[:n], V[:n], sel)
        check_attention(o[i], ref, 1e-2)


@pytest.mark.timeout(900)
def test_prefill_full_size_qwen_shape(gpu_lib):
    """A 512-query chunk at the Qwen2-7B shape (28/4 heads: seven query heads
    per KV head, laid out as eight slots), 65536 keys, top-4096: every row's
    selection is the exact top-k of its vote row; 32 rows, the first and last
    included, against the oracle's votes and decided-token rule, and the
    chunk's sparse attention on those rows against the oracle's."""
    from dataclasses import replace
    ts = gpu_lib
    cfg = replace(W.PREFILL_64K, name="prefill-512x64k-qwen2-7b-shape", num_q_heads=28,
                  num_kv_heads=4, seed=42)
    x = W.gen_prefill(cfg, device="cuda")
    q0 = x["q_pos0"]
    votes, idx = ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k)
    torch.cuda.synchronize()
    V32 = np32(votes)
    gi = idx.cpu().numpy()
    for r in range(cfg.chunk):
        n = q0 + r + 1
        assert (V32[r, n:] == 0).all()
        assert np.array_equal(gi[r], O.top_k(V32[r, :n].astype(np.float64), cfg.k)), f"row {r}"
    rows = sorted(set(np.linspace(0, cfg.chunk - 1, 32).round().astype(int).tolist()))
    Q, K = np64(x["q"]), np64(x["k_cache"])
    for r, ref in zip(rows, O.prefill_votes(Q, K, q0, rows=rows)):
        _check_votes(votes[r], ref, q0 + r + 1, cfg.num_q_heads)
        check_selection(gi[r], ref, cfg.k)
    # the chunk's sparse attention at this shape, on the same 32 rows
    from tests.parity import check_attention
    out = ts.sparse_attend_prefill(x["q"], x["k_cache"], x["v_cache"], q0, idx)
    torch.cuda.synchronize()
    o, V = np64(out), np64(x["v_cache"])
    for r in rows:
        n = q0 + r + 1
        check_attention(o[r], O.sparse_attention(Q[r], K[:n], V[:n], gi[r]), 1e-2)


@pytest.mark.timeout(900)
def test_prefill_sparse_attention_full_size(gpu_lib):
    """512 x 65536, top-4096 per query: every row's output against the
    oracle's attention over that row's own selection."""
    from tests.parity import check_attention
    ts = gpu_lib
    cfg = W.PREFILL_64K
    x = W.gen_prefill(cfg, device="cuda")
    q0 = x["q_pos0"]
    _, idx = ts.select_prefill(x["q"], x["k_cache"], q0, cfg.k)
    out = ts.sparse_attend_prefill(x["q"], x["k_cache"], x["v_cache"], q0, idx)
    torch.cuda.synchronize()
    Q, K, V = np64(x["q"]), np64(x["k_cache"]), np64(x["v_cache"])
    gi, o = idx.cpu().numpy(), np64(out)
    for i in range(cfg.chunk):
        n = q0 + i + 1
        check_attention(o[i], O.sparse_attention(Q[i], K[:n], V[:n], gi[i]), 1e-2)
