"""Pins of the fp64 oracle against things other than itself.

Each pin is a plain function that raises AssertionError when the oracle is
wrong. The ordinary tests call them; ``test_planted_mistakes`` swaps a
plausible mistake into the oracle (on the CPU) and checks that some pin
fails, so that every pin set is shown to have teeth.

What pins what:
  * worked example: hand-derived values of logits/softmax/vote/top-k/attention;
  * k = N: the whole path equals full softmax attention computed by torch's
    scaled_dot_product_attention in float64 with its own GQA convention;
  * Hq = Hkv = 1: the vote is monotone in the logit, so the selection is a
    stable library argsort of the raw dot products;
  * brute force: the chosen set maximises the vote sum over all k-subsets;
  * invariants: per-head softmax sums to 1, votes sum to Hq, attention is
    invariant under a permutation of the selected rows;
  * planted / heavy keys of the synthetic workloads are selected;
  * Selection Cache: hand-derived decisions on a circle of queries, theta
    extremes, repeated queries, the jump schedule of the drifting-query run;
  * prefill: a one-query chunk equals a decode selection; causality.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ts_oracle as O
from tests import golden
import workloads as W


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_case(seed, Hq, Hkv, d, N):
    r = _rng(seed)
    q = r.standard_normal((Hq, d))
    K = r.standard_normal((N, Hkv, d))
    V = r.standard_normal((N, Hkv, d))
    return q, K, V


SHAPES = [(1, 1, 4, 1), (2, 1, 2, 5), (4, 2, 16, 33), (7, 1, 8, 17), (8, 8, 16, 40),
          (28, 4, 32, 64), (4, 4, 64, 9)]


# ----------------------------------------------------------------------------- pins

def pin_worked_example():
    g = golden.load("worked_example.txt")
    q = np.array(g["q"]).reshape(2, 2)
    K = np.array(g["K"]).reshape(3, 1, 2)
    V = np.array(g["V"]).reshape(3, 1, 2)
    S, v = O.select(q, K, 2)
    np.testing.assert_allclose(v, g["votes"], rtol=0, atol=1e-14)
    assert list(S) == [int(x) for x in g["S_k2"]]
    np.testing.assert_allclose(O.sparse_attention(q, K, V, S).ravel(), g["out_k2"], atol=1e-14)
    S3, _ = O.select(q, K, 3)
    assert list(S3) == [int(x) for x in g["S_k3"]]
    np.testing.assert_allclose(O.sparse_attention(q, K, V, S3).ravel(), g["out_k3"], atol=1e-14)
    S1, _ = O.select(q, K, 1)
    assert list(S1) == [int(x) for x in g["S_k1"]]
    np.testing.assert_allclose(O.sparse_attention(q, K, V, S1).ravel(), g["out_k1"], atol=1e-14)
    S5, _ = O.select(q, K, 5)
    assert list(S5) == [int(x) for x in g["S_k5"]]


def pin_full_attention():
    """k = N: selection keeps every token, so the result is full attention."""
    for i, (Hq, Hkv, d, N) in enumerate(SHAPES):
        q, K, V = _rand_case(100 + i, Hq, Hkv, d, N)
        S, _ = O.select(q, K, N)
        assert sorted(S.tolist()) == list(range(N))
        out = O.sparse_attention(q, K, V, S)
        tq = torch.from_numpy(q)[None, :, None, :]                 # [1][Hq][1][d]
        tk = torch.from_numpy(K).permute(1, 0, 2)[None]            # [1][Hkv][N][d]
        tv = torch.from_numpy(V).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, scale=1.0 / math.sqrt(d), enable_gqa=(Hq != Hkv))[0, :, 0, :].numpy()
        np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def pin_softmax_and_vote_sums():
    for i, (Hq, Hkv, d, N) in enumerate(SHAPES):
        q, K, _ = _rand_case(200 + i, Hq, Hkv, d, N)
        p = O.head_softmax(O.logits(q, K))
        np.testing.assert_allclose(p.sum(axis=1), np.ones(Hq), atol=1e-12)
        v = O.soft_vote(p)
        assert abs(v.sum() - Hq) < 1e-11 * Hq
        assert (v >= 0).all()


def pin_single_head_argsort():
    """Hq = Hkv = 1: the selection is a stable argsort of the raw dot products."""
    for seed, (d, N, k) in enumerate([(4, 50, 7), (16, 300, 64), (8, 20, 20), (8, 20, 33)]):
        r = _rng(300 + seed)
        q = r.standard_normal((1, d))
        K = r.standard_normal((N, 1, d))
        raw = K[:, 0, :] @ q[0]
        want = np.sort(np.argsort(-raw, kind="stable")[:min(k, N)])
        S, _ = O.select(q, K, k)
        assert list(S[:min(k, N)]) == list(want)
        assert (S[min(k, N):] == -1).all()


def pin_bruteforce_subsets():
    """The chosen set maximises the total vote over all k-subsets (no ties)."""
    import itertools
    for seed in range(6):
        r = _rng(400 + seed)
        Hq, Hkv, d = [(2, 1, 4), (4, 2, 3), (3, 3, 2)][seed % 3]
        N = 7 + seed % 3
        q = r.standard_normal((Hq, d))
        K = r.standard_normal((N, Hkv, d))
        p = np.exp(O.logits(q, K) - O.logits(q, K).max(axis=1, keepdims=True))
        v_ref = (p / p.sum(axis=1, keepdims=True)).sum(axis=0)
        for k in (1, 3, N - 1):
            best = max(itertools.combinations(range(N), k), key=lambda c: v_ref[list(c)].sum())
            S, v = O.select(q, K, k)
            assert tuple(S) == tuple(sorted(best))


def pin_permutation_invariance():
    for i, (Hq, Hkv, d, N) in enumerate(SHAPES[2:]):
        q, K, V = _rand_case(500 + i, Hq, Hkv, d, N)
        r = _rng(600 + i)
        S = np.sort(r.choice(N, size=max(1, N // 3), replace=False))
        out = O.sparse_attention(q, K, V, S)
        out_perm = O.sparse_attention(q, K, V, r.permutation(S))
        np.testing.assert_allclose(out, out_perm, rtol=1e-12, atol=1e-13)
        perm = r.permutation(N)          # move rows; remap the indices
        inv = np.argsort(perm)
        out_moved = O.sparse_attention(q, K[perm], V[perm], inv[S])
        np.testing.assert_allclose(out, out_moved, rtol=1e-12, atol=1e-13)


def pin_uniform_ties():
    """q = 0: every logit is 0, votes are Hq/N, ties keep the lowest indices."""
    Hq, Hkv, d, N = 4, 2, 8, 10
    q = np.zeros((Hq, d))
    K = _rng(7).standard_normal((N, Hkv, d))
    S, v = O.select(q, K, 4)
    np.testing.assert_allclose(v, np.full(N, Hq / N), atol=1e-15)
    assert list(S) == [0, 1, 2, 3]


def pin_planted_tokens():
    cfg = W.TINY
    x = W.gen_decode(cfg)
    q = x["q"][0].double().numpy()
    K = x["k_cache"][0].double().numpy()
    S, _ = O.select(q, K, cfg.k)
    assert set(x["special"][0].tolist()) <= set(S.tolist())


def pin_heavy_tokens():
    cfg = W.QWEN_32K
    x = W.gen_decode(cfg)
    q = x["q"][0].float().double().numpy()
    K = x["k_cache"][0].float().double().numpy()
    S, v = O.select(q, K, cfg.k)
    heavy = x["special"][0].tolist()
    assert len(heavy) == 327
    assert set(heavy) <= set(S.tolist())
    assert abs(v.sum() - cfg.num_q_heads) < 1e-9


def _circle_queries(steps, cos_a):
    a = math.acos(cos_a)
    return [np.array([[math.cos(t * a), math.sin(t * a)]]) for t in range(steps)]


def pin_selcache_circle():
    g = golden.load("selcache_example.txt")
    steps = int(g["steps"][0])
    qs = _circle_queries(steps, g["cos_a"][0])
    K = _rng(8).standard_normal((6, 1, 2))
    V = _rng(9).standard_normal((6, 1, 2))
    cases = [(0, 0.9, "hits_mode0_theta0.9"), (1, 0.9, "hits_mode1_theta0.9"),
             (0, 1.0, "hits_theta1.0"), (1, 1.0, "hits_theta1.0"),
             (0, -1.5, "hits_theta-1.5"), (1, -1.5, "hits_theta-1.5")]
    for mode, theta, key in cases:
        _, _, hits, _ = O.run_decode(qs, K, V, 3, theta, mode)
        assert [int(h) for h in hits] == [int(x) for x in g[key]], (mode, theta)


def pin_selcache_reuse():
    """A hit returns the previous selection unchanged even though q moved."""
    Hq, Hkv, d, N = 4, 2, 8, 64
    q, K, V = _rand_case(10, Hq, Hkv, d, N)
    cache = O.SelectionCache(0)
    _, S0, h0, _ = cache.step(q, K, V, 8, 0.5)
    q2 = q + 0.05 * _rng(11).standard_normal(q.shape)
    out, S1, h1, c = cache.step(q2, K, V, 8, 0.5)
    assert not h0 and h1 and c > 0.5
    assert list(S1) == list(S0)
    np.testing.assert_allclose(out, O.sparse_attention(q2, K, V, S0), atol=1e-14)
    # the same query again always hits for theta < 1
    _, _, h2, c2 = cache.step(q2, K, V, 8, 0.999999)
    assert h2 and abs(c2 - 1.0) < 1e-12
    # theta >= 1 never hits: the run equals the no-cache run
    outs, sels, hits, _ = O.run_decode([q, q, q2], K, V, 8, 1.0)
    assert not hits.any()
    for t, qq in enumerate([q, q, q2]):
        assert list(sels[t]) == list(O.select(qq, K, 8)[0])


def pin_selcache_jump_schedule():
    """Drifting queries (keep 0.95, noise 0.31) with a jump every 32 steps:
    consecutive cosines sit near 0.95 and jumps near 0, so at theta = 0.9
    mode 0 misses exactly at t = 0, 32, 64, ..."""
    steps = 96
    Q = W.gen_query_process(steps, 2, 32, 128, seed=5).to(torch.bfloat16).double().numpy()
    K = _rng(12).standard_normal((16, 8, 128))
    V = _rng(13).standard_normal((16, 8, 128))
    for b in range(2):
        _, _, hits, cos = O.run_decode(Q[:, b], K, V, 4, 0.9, 0)
        misses = [t for t in range(steps) if not hits[t]]
        assert misses == list(range(0, steps, 32))
        inner = [c for t, c in enumerate(cos) if t % 32]
        assert 0.93 < min(inner) and max(inner) < 0.97


def pin_prefill_one_query_is_decode():
    Hq, Hkv, d, n = 8, 2, 16, 50
    r = _rng(14)
    Q = r.standard_normal((5, Hq, d))
    K = r.standard_normal((n, Hkv, d))
    q_pos0 = n - 5
    rows = O.prefill_select(Q, K, q_pos0, 6)
    for i in range(5):
        want, _ = O.select(Q[i], K[:q_pos0 + i + 1], 6)
        assert list(rows[i]) == list(want)
        assert rows[i].max() <= q_pos0 + i
    votes = O.prefill_votes(Q, K, q_pos0)
    for i, v in enumerate(votes):
        assert v.shape == (q_pos0 + i + 1,)
        assert abs(v.sum() - Hq) < 1e-11


def pin_edge_cases():
    q, K, V = _rand_case(15, 4, 2, 8, 5)
    S, _ = O.select(q, K, 9)            # k > N
    assert list(S) == [0, 1, 2, 3, 4, -1, -1, -1, -1]
    empty = K[:0]
    S0, v0 = O.select(q, empty, 3)
    assert list(S0) == [-1, -1, -1] and v0.shape == (0,)
    assert (O.sparse_attention(q, empty, V[:0], S0) == 0).all()
    cache = O.SelectionCache(0)
    out, S1, hit, _ = cache.step(q, empty, V[:0], 3, -2.0)
    assert not hit and not cache.valid and (out == 0).all()


def pin_paged_layout():
    """The paged-layout helper against a hand-written pool whose rows name
    their own (page, slot): a shuffled page table, an unused pool page and a
    partial last page (tests/golden/paged_layout.txt)."""
    g = golden.load("paged_layout.txt")
    P, npages = int(g["page_size"][0]), int(g["pages"][0])
    pool = np.zeros((npages, P, 1, 2))
    for pg in range(npages):
        for s in range(P):
            pool[pg, s, 0] = [10 * pg + s, -(10 * pg + s)]
    pt = np.array([int(x) for x in g["page_table"]])
    rows = O.paged_to_contiguous(pool, pt, int(g["n"][0]))
    assert rows.shape == (int(g["n"][0]), 1, 2)
    assert rows[:, 0, 0].tolist() == g["rows_ch0"]
    assert rows[:, 0, 1].tolist() == g["rows_ch1"]
    short = O.paged_to_contiguous(pool, pt, int(g["n_short"][0]))
    assert short[:, 0, 0].tolist() == g["rows_short_ch0"]


PINS = {name: fn for name, fn in list(globals().items()) if name.startswith("pin_")}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name]()


# ------------------------------------------------------------------ planted mistakes

def _mut_scale(d):
    return 1.0


def _mut_kv_head(h, G):
    return h % G


def _mut_softmax_axis(s):
    if s.shape[1] == 0:
        return s.copy()
    m = s.max(axis=0, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=0, keepdims=True)


def _mut_vote_max(p):
    return p.max(axis=0)


def _mut_vote_logits(p):
    return np.log(np.maximum(p, 1e-300)).sum(axis=0)


def _mut_tie_high(v, k):
    N = v.shape[0]
    k_eff = min(k, N)
    order = np.lexsort((-np.arange(N), -v))
    out = np.full(k, -1, dtype=np.int64)
    out[:k_eff] = np.sort(order[:k_eff])
    return out


def _mut_unsorted(v, k):
    N = v.shape[0]
    k_eff = min(k, N)
    order = np.lexsort((np.arange(N), -v))
    out = np.full(k, -1, dtype=np.int64)
    out[:k_eff] = order[:k_eff]
    return out


def _mut_keff(v, k):
    N = v.shape[0]
    k_eff = max(0, min(k, N) - 1)
    order = np.lexsort((np.arange(N), -v))
    out = np.full(k, -1, dtype=np.int64)
    out[:k_eff] = np.sort(order[:k_eff])
    return out


_orig_attention = O.sparse_attention


def _mut_attend_all(q, K, V, S, scale=None):
    if np.asarray(S)[np.asarray(S) >= 0].size == 0:
        return _orig_attention(q, K, V, S, scale)
    return _orig_attention(q, K, V, np.arange(K.shape[0]), scale)


def _mut_attend_v_is_k(q, K, V, S, scale=None):
    return _orig_attention(q, K, K, S, scale)


_orig_logits = O.logits


def _mut_logit_sign(q, K, scale=None):
    return -_orig_logits(q, K, scale)


class _MutCacheGe(O.SelectionCache):
    def decide(self, q, theta):
        if not self.valid:
            return False, float("nan")
        c = O.cosine(q, self.prev_q)
        return bool(c >= theta), c


class _MutCacheAnchorAlways(O.SelectionCache):
    def step(self, q, K, V, k, theta, scale=None):
        self.mode = 0
        return super().step(q, K, V, k, theta, scale)


class _MutCacheNoUpdate(O.SelectionCache):
    """Keeps the first query forever (never updates prev_q)."""
    def step(self, q, K, V, k, theta, scale=None):
        keep = self.prev_q
        out = super().step(q, K, V, k, theta, scale)
        if keep is not None:
            self.prev_q = keep
        return out


_orig_prefill_votes = O.prefill_votes


def _mut_prefill_offbyone(Q, K, q_pos0, rows=None, scale=None):
    rows = range(Q.shape[0]) if rows is None else rows
    return [O.soft_vote(O.head_softmax(O.logits(Q[i], K[:max(1, q_pos0 + i)], scale)))
            for i in rows]


def _mut_paged_swapped(pool, page_table_row, n):
    P = pool.shape[1]
    j = np.arange(n)
    return pool[page_table_row[j % P], j // P]


MUTANTS = {
    "paged_page_slot_swapped": ("paged_to_contiguous", _mut_paged_swapped),
    "scale_dropped": ("default_scale", _mut_scale),
    "gqa_map_modulo": ("kv_head_of", _mut_kv_head),
    "softmax_over_heads": ("head_softmax", _mut_softmax_axis),
    "vote_max_not_sum": ("soft_vote", _mut_vote_max),
    "vote_of_log_probs": ("soft_vote", _mut_vote_logits),
    "ties_to_higher_index": ("top_k", _mut_tie_high),
    "indices_not_sorted": ("top_k", _mut_unsorted),
    "k_eff_off_by_one": ("top_k", _mut_keff),
    "attend_all_tokens": ("sparse_attention", _mut_attend_all),
    "value_is_key": ("sparse_attention", _mut_attend_v_is_k),
    "logit_sign": ("logits", _mut_logit_sign),
    "cache_ge_theta": ("SelectionCache", _MutCacheGe),
    "cache_mode1_moves_anchor": ("SelectionCache", _MutCacheAnchorAlways),
    "cache_never_updates_q": ("SelectionCache", _MutCacheNoUpdate),
    "prefill_causal_off_by_one": ("prefill_votes", _mut_prefill_offbyone),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistakes(mutant, monkeypatch):
    attr, repl = MUTANTS[mutant]
    monkeypatch.setattr(O, attr, repl)
    failed = []
    for name, fn in PINS.items():
        if name in ("pin_heavy_tokens",):        # slow; covered by the others
            continue
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    assert failed, f"no pin caught the planted mistake {mutant}"
