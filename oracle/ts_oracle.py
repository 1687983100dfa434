"""Plain fp64 CPU oracle of TokenSelect's token selection and sparse attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module. The HIP path
never calls it, and it shares no code with the HIP path: it imports NumPy
and nothing else.

Sources (the pages given for this method):
  * TokenSelect README ("TokenSelect: Efficient Long-Context Inference and
    Length Extrapolation for LLMs via Dynamic Token-Level KV Cache
    Selection", GitHub page), section "Key Takeaways": each cached token's
    importance is measured per head by the dot product of the query with its
    key; per-head soft voting (softmax per head, then a sum over heads); the
    Selection Cache, by which similar queries in a row reuse one selection;
    and attention restricted to the few selected tokens.
  * GrooveSquid summary of the same paper, "Medium Difficulty Summary":
    the same three parts (per-head soft voting, Selection Cache, a dot
    product kernel).
  * The method statement this build follows fixes what the pages leave
    open: the 1/sqrt(d) scale, grouped-query attention (each KV head serves
    a contiguous group of query heads), a softmax over all N cached tokens,
    reuse when the cosine of consecutive queries exceeds theta, and a
    chunked-prefill variant that is causal within the chunk.

Every floating-point step runs in float64. Stored inputs (bf16 or fp32) are
upcast exactly by the caller before they reach these functions.

Readings where the pages are silent (each is a parameter or documented rule):
  R1  scale tau = 1/sqrt(d) unless given.
  R2  kv head of query head h is floor(h / G), G = Hq / Hkv.
  R3  each head's softmax runs over all N cached tokens; no sink/window.
  R4  k_eff = min(k, N); the selection is padded with -1 up to k.
  R5  ties at the k-th vote go to the lower token index.
  R6  indices are returned in ascending order.
  R7  attention renormalises over the selected tokens only, with the same tau;
      one selection is shared by every head of the sequence.
  R8  the Selection Cache compares the flattened (Hq*d) query with the
      previous step's query (mode 0), or with the query of the last miss
      (mode 1, "anchor"); a hit needs valid state and cos > theta strictly;
      a zero-norm query or previous query never hits; the first step and a
      step on an empty sequence are misses, and an empty sequence leaves the
      state invalid.
  R9  prefill query i of a chunk sits at absolute position q_pos0+i and sees
      keys 0 .. q_pos0+i; its vote row has length q_pos0+i+1.

Pins: every function here is checked in tests/test_oracle.py against
textbook results (full attention when k = N, a library sort when Hq = Hkv =
1, exhaustive subset search on tiny inputs), invariants (per-head softmax
sums to 1, votes sum to Hq, permutation invariance), a hand-derived worked
example (tests/golden/worked_example.txt), closed forms of the
selection-cache decisions, a hand-written paged pool for the paged-layout
helper (tests/golden/paged_layout.txt), and planted-mistake tests.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "group_size", "kv_head_of", "default_scale", "logits", "head_softmax", "soft_vote",
    "top_k", "select", "sparse_attention", "cosine", "SelectionCache", "run_decode",
    "prefill_votes", "prefill_select", "paged_to_contiguous",
]


def group_size(num_q_heads: int, num_kv_heads: int) -> int:
    """G = Hq / Hkv; grouped-query attention needs Hkv to divide Hq (reading R2)."""
    if num_kv_heads <= 0 or num_q_heads % num_kv_heads != 0:
        raise ValueError("num_q_heads must be a positive multiple of num_kv_heads")
    return num_q_heads // num_kv_heads


def kv_head_of(h: int, G: int) -> int:
    """KV head serving query head h: contiguous groups of G query heads (R2)."""
    return h // G


def default_scale(d: int) -> float:
    """tau = 1/sqrt(d) (R1)."""
    return 1.0 / math.sqrt(d)


def logits(q: np.ndarray, K: np.ndarray, scale: float | None = None) -> np.ndarray:
    """Per-head token criticality: s[h, j] = tau * <q[h], K[j, kv(h)]>.

    README "Key Takeaways", first point (per-head dot product of query and
    key, one value per cached token). q [Hq][d], K [N][Hkv][d], both
    float64 -> s [Hq][N].
    """
    Hq, d = q.shape
    N, Hkv, dk = K.shape
    assert dk == d
    G = group_size(Hq, Hkv)
    tau = default_scale(d) if scale is None else scale
    s = np.empty((Hq, N), dtype=np.float64)
    for h in range(Hq):
        s[h] = tau * (K[:, kv_head_of(h, G), :] @ q[h])
    return s


def head_softmax(s: np.ndarray) -> np.ndarray:
    """p[h, j] = exp(s[h, j] - m_h) / sum_j' exp(s[h, j'] - m_h), over all N tokens.

    README "Key Takeaways", second point (normalise each head's criticality
    through softmax); R3. s [Hq][N] -> p [Hq][N].
    """
    if s.shape[1] == 0:
        return s.copy()
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def soft_vote(p: np.ndarray) -> np.ndarray:
    """v[j] = sum_h p[h, j]: per-head soft voting, an unweighted sum over heads.

    README "Key Takeaways", second point; GrooveSquid medium summary.
    """
    return p.sum(axis=0)


def top_k(v: np.ndarray, k: int) -> np.ndarray:
    """The k_eff = min(k, N) tokens with the largest votes (R4-R6).

    Order: vote descending, then index ascending, so the lower index wins a
    tie. The chosen set is returned ascending and padded with -1 to length k.
    README "Key Takeaways" (attention keeps only a few selected tokens).
    """
    N = v.shape[0]
    k_eff = min(k, N)
    order = np.lexsort((np.arange(N), -v))
    out = np.full(k, -1, dtype=np.int64)
    out[:k_eff] = np.sort(order[:k_eff])
    return out


def select(q: np.ndarray, K: np.ndarray, k: int, scale: float | None = None):
    """Scoring, per-head softmax, soft vote and top-k for one decode query.

    Returns (indices [k], votes [N]).
    """
    v = soft_vote(head_softmax(logits(q, K, scale)))
    return top_k(v, k), v


def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, S: np.ndarray,
                     scale: float | None = None) -> np.ndarray:
    """Softmax attention of every query head over the selected tokens only (R7).

    README "Key Takeaways" (the attention sees the selected tokens only).
    q [Hq][d], K/V [N][Hkv][d], S indices (-1 = padding, ignored) -> out
    [Hq][d]. An empty selection gives zeros.
    """
    Hq, d = q.shape
    _, Hkv, _ = K.shape
    G = group_size(Hq, Hkv)
    tau = default_scale(d) if scale is None else scale
    sel = np.asarray(S)
    sel = sel[sel >= 0]
    out = np.zeros((Hq, V.shape[2]), dtype=np.float64)
    if sel.size == 0:
        return out
    for h in range(Hq):
        g = kv_head_of(h, G)
        s = tau * (K[sel, g, :] @ q[h])
        w = np.exp(s - s.max())
        w = w / w.sum()
        out[h] = w @ V[sel, g, :]
    return out


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    """Cosine similarity of two flattened query vectors; NaN if either norm is 0."""
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na = math.sqrt(float(a @ a))
    nb = math.sqrt(float(b @ b))
    if na == 0.0 or nb == 0.0:
        return float("nan")
    return float(a @ b) / (na * nb)


class SelectionCache:
    """Selection-cache state of one sequence (one layer), reading R8.

    README "Key Takeaways", third point: when successive queries are alike,
    the earlier selection is reused, so selection runs less often.
    """

    def __init__(self, mode: int = 0):
        assert mode in (0, 1)
        self.mode = mode
        self.reset()

    def reset(self):
        self.valid = False
        self.prev_q = None
        self.prev_S = None

    def decide(self, q: np.ndarray, theta: float) -> tuple[bool, float]:
        """(hit, cos) for query q against the stored query."""
        if not self.valid:
            return False, float("nan")
        c = cosine(q, self.prev_q)
        return bool(c > theta), c          # NaN > theta is False: a miss

    def step(self, q: np.ndarray, K: np.ndarray, V: np.ndarray, k: int, theta: float,
             scale: float | None = None):
        """One decode step: returns (out [Hq][d], S [k], hit, cos)."""
        N = K.shape[0]
        hit, c = self.decide(q, theta)
        if N == 0:
            hit = False
        if hit:
            S = self.prev_S
        else:
            S, _ = select(q, K, k, scale)
        out = sparse_attention(q, K, V, S, scale)
        if N == 0:
            self.reset()
            return out, S, False, c
        if self.mode == 0 or not hit:
            self.prev_q = np.array(q, dtype=np.float64, copy=True)
        self.prev_S = S
        self.valid = True
        return out, S, hit, c


def run_decode(queries, K, V, k: int, theta: float, mode: int = 0, scale: float | None = None):
    """A run of decode steps of one sequence over a fixed cache.

    queries [T][Hq][d] -> (outs [T][Hq][d], S [T][k], hits [T] bool, cos [T]).
    """
    cache = SelectionCache(mode)
    outs, sels, hits, coss = [], [], [], []
    for q in queries:
        o, S, h, c = cache.step(q, K, V, k, theta, scale)
        outs.append(o)
        sels.append(S)
        hits.append(h)
        coss.append(c)
    return np.array(outs), np.array(sels), np.array(hits), np.array(coss)


def prefill_votes(Q: np.ndarray, K: np.ndarray, q_pos0: int, rows=None,
                  scale: float | None = None) -> list:
    """Soft-vote rows of a prefill chunk, causal within the chunk (R9).

    Q [C][Hq][d], K [n_ctx][Hkv][d]. Query i sees keys j <= q_pos0 + i. Returns
    a list of vote rows (row i has length q_pos0 + i + 1) for the requested rows.
    """
    C = Q.shape[0]
    rows = range(C) if rows is None else rows
    out = []
    for i in rows:
        n_i = q_pos0 + i + 1
        out.append(soft_vote(head_softmax(logits(Q[i], K[:n_i], scale))))
    return out


def prefill_select(Q: np.ndarray, K: np.ndarray, q_pos0: int, k: int, rows=None,
                   scale: float | None = None) -> np.ndarray:
    """Top-k selection of each prefill query's own vote row -> [len(rows)][k]."""
    votes = prefill_votes(Q, K, q_pos0, rows, scale)
    return np.array([top_k(v, k) for v in votes])


def paged_to_contiguous(pool: np.ndarray, page_table_row: np.ndarray, n: int) -> np.ndarray:
    """Token j of a paged sequence lives at pool[page_table_row[j // P], j % P]."""
    P = pool.shape[1]
    j = np.arange(n)
    return pool[page_table_row[j // P], j % P]
