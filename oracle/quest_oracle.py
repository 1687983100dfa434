"""Plain fp64 CPU oracle of Quest-style page selection (an alternative selector).

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module. The HIP path never
calls it and shares no code with it.

Source: the page on "Quest: Query-Aware Sparsity for Efficient Long-Context
LLM Inference" (bohrium.dp.tech, arXiv 2406.10774): its abstract, and point 4
of its "Method Overview". The KV cache is cut into pages. Each page keeps the
channel-wise minimum and maximum of its keys. A page's criticality is
estimated from the current query's element-wise products with those two
vectors, and only the Top-K pages take part in attention.

Readings where the page is silent:
  Q1  Per channel c the larger of q_c*min_c and q_c*max_c is kept and the
      channels are summed: the estimate is then an upper bound of q.k for
      every key k of the page (the reason to keep both extremes), scaled by
      tau = 1/sqrt(d) like the logits.
  Q2  Grouped-query attention: a KV head's page score is the largest estimate
      over the query heads of its group, so a page stays if any head that
      reads it could rate one of its keys highly; each KV head keeps its own
      Top-K pages, and every query head attends over all valid tokens of its
      KV head's pages (softmax renormalised over them, scale tau).
  Q3  Pages are the KV cache's own pages (page size P); logical page i holds
      tokens iP .. iP+P-1 that exist (the last page may be partial; its
      extremes run over its existing tokens only).
  Q4  K_pages = min(K, number of pages); ties go to the lower page index and
      pages are listed ascending, padded with -1 (as in the token top-k).

Every floating-point step runs in float64 on exactly upcast stored values.
Pins: tests/test_oracle.py checks the upper-bound property against brute force
over every key, equality for one-token pages with one head per group, the
group maximum against brute force, a planted page, and full attention when
every page is kept.
"""
from __future__ import annotations

import numpy as np

from oracle.ts_oracle import default_scale, group_size, kv_head_of, top_k

__all__ = ["page_extremes", "page_scores", "select_pages", "pages_to_tokens",
           "page_attention"]


def page_extremes(K: np.ndarray, page_size: int):
    """Channel-wise min and max keys of each page (Q3).

    K [N][Hkv][d] -> (kmin, kmax), each [n_pages][Hkv][d], n_pages = ceil(N/P).
    """
    N, Hkv, d = K.shape
    n_pages = -(-N // page_size)
    kmin = np.empty((n_pages, Hkv, d), dtype=np.float64)
    kmax = np.empty((n_pages, Hkv, d), dtype=np.float64)
    for i in range(n_pages):
        rows = K[i * page_size:min(N, (i + 1) * page_size)]
        kmin[i] = rows.min(axis=0)
        kmax[i] = rows.max(axis=0)
    return kmin, kmax


def page_scores(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray,
                scale: float | None = None) -> np.ndarray:
    """Criticality estimate of every page for every KV head (Q1, Q2).

    q [Hq][d] -> [Hkv][n_pages]: for KV head g, the largest over the query
    heads h of g's group of tau * sum_c max(q[h,c]*kmin[.,g,c], q[h,c]*kmax[.,g,c]).
    """
    Hq, d = q.shape
    n_pages, Hkv, _ = kmin.shape
    G = group_size(Hq, Hkv)
    tau = default_scale(d) if scale is None else scale
    out = np.full((Hkv, n_pages), -np.inf, dtype=np.float64)
    for h in range(Hq):
        g = kv_head_of(h, G)
        est = tau * np.maximum(kmin[:, g, :] * q[h], kmax[:, g, :] * q[h]).sum(axis=1)
        out[g] = np.maximum(out[g], est)
    return out


def select_pages(q: np.ndarray, K: np.ndarray, page_size: int, k_pages: int,
                 scale: float | None = None):
    """Top-K pages per KV head (Q4): returns (pages [Hkv][k_pages], scores [Hkv][n_pages])."""
    kmin, kmax = page_extremes(K, page_size)
    s = page_scores(q, kmin, kmax, scale)
    return np.array([top_k(row, k_pages) for row in s]), s


def pages_to_tokens(pages: np.ndarray, page_size: int, n: int) -> np.ndarray:
    """The existing tokens of a list of logical pages (-1 entries ignored), ascending."""
    pg = np.asarray(pages)
    pg = np.sort(pg[pg >= 0])
    if pg.size == 0:
        return np.zeros(0, dtype=np.int64)
    tok = (pg[:, None] * page_size + np.arange(page_size)[None, :]).ravel()
    return tok[tok < n]


def page_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, pages: np.ndarray,
                   page_size: int, scale: float | None = None) -> np.ndarray:
    """Attention of every query head over the tokens of its KV head's pages (Q2).

    pages [Hkv][k_pages] (-1 = padding) -> out [Hq][d]; no page gives zeros.
    """
    Hq, d = q.shape
    N, Hkv, _ = K.shape
    G = group_size(Hq, Hkv)
    tau = default_scale(d) if scale is None else scale
    out = np.zeros((Hq, V.shape[2]), dtype=np.float64)
    for h in range(Hq):
        g = kv_head_of(h, G)
        tok = pages_to_tokens(pages[g], page_size, N)
        if tok.size == 0:
            continue
        s = tau * (K[tok, g, :] @ q[h])
        w = np.exp(s - s.max())
        out[h] = (w / w.sum()) @ V[tok, g, :]
    return out
