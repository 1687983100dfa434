"""Pins of the Quest page-selection oracle against things other than itself.

  * box maximum: a page's estimate equals the largest q.x over every corner x
    of the box [min, max] of its keys, enumerated corner by corner (d small);
  * upper bound: the estimate is >= tau * q.k for every key of the page, by
    brute force over all keys and heads;
  * one-token pages: the estimate is exactly the largest logit of the group;
  * planted page: a page holding a key along a head's query is selected;
  * every page kept: page attention equals torch's full attention;
  * one-token pages and one shared page set: page attention equals the
    (separately pinned) token-level sparse attention;
  * hand examples of the page extremes and of the page-to-token expansion.
``test_quest_planted_mistakes`` swaps plausible mistakes into the oracle and
checks that some pin fails.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import quest_oracle as Q
from oracle import ts_oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, Hq, Hkv, d, N):
    r = _rng(seed)
    return (r.standard_normal((Hq, d)), r.standard_normal((N, Hkv, d)),
            r.standard_normal((N, Hkv, d)))


SHAPES = [  # Hq, Hkv, d, N, page_size
    (1, 1, 3, 7, 2), (4, 2, 3, 13, 4), (4, 1, 2, 9, 3), (8, 8, 3, 16, 16), (6, 2, 4, 11, 5)]


def pin_box_maximum():
    for i, (Hq, Hkv, d, N, P) in enumerate(SHAPES):
        q, K, _ = _case(10 + i, Hq, Hkv, d, N)
        kmin, kmax = Q.page_extremes(K, P)
        s = Q.page_scores(q, kmin, kmax)
        G = Hq // Hkv
        tau = 1.0 / math.sqrt(d)
        for g in range(Hkv):
            for p in range(kmin.shape[0]):
                best = -math.inf
                for h in range(g * G, (g + 1) * G):
                    for corner in itertools.product((0, 1), repeat=d):
                        x = [kmax[p, g, c] if corner[c] else kmin[p, g, c] for c in range(d)]
                        best = max(best, tau * sum(q[h, c] * x[c] for c in range(d)))
                assert abs(s[g, p] - best) <= 1e-12 * max(1.0, abs(best)), (i, g, p)


def pin_upper_bound():
    for i, (Hq, Hkv, d, N, P) in enumerate(SHAPES + [(28, 4, 32, 100, 16)]):
        q, K, _ = _case(20 + i, Hq, Hkv, d, N)
        s = Q.page_scores(q, *Q.page_extremes(K, P))
        G = Hq // Hkv
        tau = 1.0 / math.sqrt(d)
        for j in range(N):
            for h in range(Hq):
                g = h // G
                assert s[g, j // P] >= tau * float(q[h] @ K[j, g]) - 1e-12


def pin_single_token_pages():
    for i, (Hq, Hkv, d, N, _) in enumerate(SHAPES):
        q, K, _ = _case(30 + i, Hq, Hkv, d, N)
        s = Q.page_scores(q, *Q.page_extremes(K, 1))
        G = Hq // Hkv
        tau = 1.0 / math.sqrt(d)
        for g in range(Hkv):
            for j in range(N):
                want = max(tau * float(q[h] @ K[j, g]) for h in range(g * G, (g + 1) * G))
                assert abs(s[g, j] - want) <= 1e-12 * max(1.0, abs(want))


def pin_extremes_hand_example():
    K = np.array([[[1.0, -2.0]], [[3.0, 0.5]], [[-1.0, 4.0]], [[2.0, 2.0]], [[0.0, -5.0]]])
    kmin, kmax = Q.page_extremes(K, 2)        # pages {0,1}, {2,3}, {4}
    assert kmin.shape == (3, 1, 2)
    assert kmin[:, 0].tolist() == [[1.0, -2.0], [-1.0, 2.0], [0.0, -5.0]]
    assert kmax[:, 0].tolist() == [[3.0, 0.5], [2.0, 4.0], [0.0, -5.0]]
    # q = (1, -1), tau = 1/sqrt(2): page 0 -> max(1,3) + max(2,-0.5) = 5
    s = Q.page_scores(np.array([[1.0, -1.0]]), kmin, kmax)
    np.testing.assert_allclose(s[0] * math.sqrt(2), [5.0, 0.0, 5.0], atol=1e-14)
    pages, _ = Q.select_pages(np.array([[1.0, -1.0]]), K, 2, 2)
    assert pages.tolist() == [[0, 2]]          # tie between pages 0 and 2 at 5: both kept
    pages, _ = Q.select_pages(np.array([[1.0, -1.0]]), K, 2, 1)
    assert pages.tolist() == [[0]]             # lower index wins the tie
    pages, _ = Q.select_pages(np.array([[1.0, -1.0]]), K, 2, 5)
    assert pages.tolist() == [[0, 1, 2, -1, -1]]


def pin_pages_to_tokens():
    assert Q.pages_to_tokens(np.array([3, -1, 0]), 4, 14).tolist() == [0, 1, 2, 3, 12, 13]
    assert Q.pages_to_tokens(np.array([-1, -1]), 4, 14).tolist() == []
    assert Q.pages_to_tokens(np.array([1]), 1, 5).tolist() == [1]


def pin_planted_page():
    Hq, Hkv, d, N, P = 8, 2, 16, 160, 16
    q, K, _ = _case(40, Hq, Hkv, d, N)
    # head 5 (KV head 1): a key along its query in page 7; head 0 (KV head 0): page 2
    K[7 * P + 3, 1] = 6.0 * q[5] / np.linalg.norm(q[5]) * math.sqrt(d)
    K[2 * P + 9, 0] = 6.0 * q[0] / np.linalg.norm(q[0]) * math.sqrt(d)
    pages, _ = Q.select_pages(q, K, P, 1)
    assert pages.tolist() == [[2], [7]]


def pin_all_pages_full_attention():
    for i, (Hq, Hkv, d, N, P) in enumerate(SHAPES):
        q, K, V = _case(50 + i, Hq, Hkv, d, N)
        n_pages = -(-N // P)
        pages, _ = Q.select_pages(q, K, P, n_pages + 2)
        out = Q.page_attention(q, K, V, pages, P)
        tq = torch.from_numpy(q)[None, :, None, :]
        tk = torch.from_numpy(K).permute(1, 0, 2)[None]
        tv = torch.from_numpy(V).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, scale=1.0 / math.sqrt(d), enable_gqa=(Hq != Hkv))[0, :, 0, :].numpy()
        np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def pin_one_token_pages_sparse_attention():
    Hq, Hkv, d, N = 8, 2, 16, 40
    q, K, V = _case(60, Hq, Hkv, d, N)
    S = np.array([1, 5, 6, 20, 39, -1])
    pages = np.stack([S, S])
    np.testing.assert_allclose(Q.page_attention(q, K, V, pages, 1),
                               O.sparse_attention(q, K, V, S), rtol=1e-12, atol=1e-13)
    # a KV head without pages gives zeros for its query heads only
    pages = np.stack([S, np.full_like(S, -1)])
    out = Q.page_attention(q, K, V, pages, 1)
    assert (out[4:] == 0).all() and (out[:4] != 0).any()


PINS = {name: fn for name, fn in list(globals().items()) if name.startswith("pin_")}


@pytest.mark.parametrize("name", sorted(PINS))
def test_quest_pin(name):
    PINS[name]()


# ------------------------------------------------------------------ planted mistakes

_orig_scores = Q.page_scores
_orig_extremes = Q.page_extremes
_orig_attention = Q.page_attention
_orig_tokens = Q.pages_to_tokens


def _mut_scores_sum_heads(q, kmin, kmax, scale=None):
    Hq, d = q.shape
    _, Hkv, _ = kmin.shape
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.zeros((Hkv, kmin.shape[0]))
    for h in range(Hq):
        out[h // G] += tau * np.maximum(kmin[:, h // G] * q[h], kmax[:, h // G] * q[h]).sum(axis=1)
    return out


def _mut_scores_max_only(q, kmin, kmax, scale=None):
    return _orig_scores(q, kmax, kmax, scale)


def _mut_scores_min_of_products(q, kmin, kmax, scale=None):
    return -_orig_scores(-q, kmin, kmax, scale)


def _mut_extremes_overlap(K, page_size):
    N = K.shape[0]
    n_pages = -(-N // page_size)
    kmin = np.empty((n_pages,) + K.shape[1:])
    kmax = np.empty((n_pages,) + K.shape[1:])
    for i in range(n_pages):
        rows = K[i * page_size:min(N, (i + 1) * page_size + 1)]
        kmin[i], kmax[i] = rows.min(axis=0), rows.max(axis=0)
    return kmin, kmax


def _mut_tokens_past_end(pages, page_size, n):
    pg = np.asarray(pages)
    pg = np.sort(pg[pg >= 0])
    return (pg[:, None] * page_size + np.arange(page_size)[None, :]).ravel()


def _mut_attention_shared_pages(q, K, V, pages, page_size, scale=None):
    return _orig_attention(q, K, V, np.stack([pages[0]] * pages.shape[0]), page_size, scale)


def _mut_tie_high(v, k):
    N = v.shape[0]
    order = np.lexsort((-np.arange(N), -v))
    out = np.full(k, -1, dtype=np.int64)
    out[:min(k, N)] = np.sort(order[:min(k, N)])
    return out


QUEST_MUTANTS = {
    "scale_dropped": ("default_scale", lambda d: 1.0),
    "gqa_map_modulo": ("kv_head_of", lambda h, G: h % G),
    "group_sum_not_max": ("page_scores", _mut_scores_sum_heads),
    "max_key_only": ("page_scores", _mut_scores_max_only),
    "lower_bound_not_upper": ("page_scores", _mut_scores_min_of_products),
    "pages_overlap": ("page_extremes", _mut_extremes_overlap),
    "tokens_past_end": ("pages_to_tokens", _mut_tokens_past_end),
    "one_page_set_for_all_heads": ("page_attention", _mut_attention_shared_pages),
    "ties_to_higher_index": ("top_k", _mut_tie_high),
}


@pytest.mark.parametrize("mutant", sorted(QUEST_MUTANTS))
def test_quest_planted_mistakes(mutant, monkeypatch):
    attr, repl = QUEST_MUTANTS[mutant]
    monkeypatch.setattr(Q, attr, repl)
    failed = []
    for name, fn in PINS.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    assert failed, f"no pin caught the planted mistake {mutant}"
