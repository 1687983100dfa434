"""Parity rules shared by the GPU tests (HIP path vs the fp64 oracle).

* Selection (index work): the GPU's set must hold exactly k_eff = min(k, N)
  distinct indices in ascending order, -1 padded; every token whose oracle vote
  lies more than 1e-5 * max(vote) from the oracle's k-th vote must be inside or
  outside the set exactly as in the oracle's set. Tokens closer than that to
  the k-th vote are ties up to rounding and may go either way.
* The top-k kernel alone is index work on given fp32 inputs: bit-exact against
  the oracle's top_k applied to the same fp32 values.
* Attention outputs: per (sequence, head), max |o - o_ref| <= tol * max |o_ref|,
  with o_ref the oracle's attention over the GPU's own selection.
"""
import numpy as np
import torch


def np32(t: torch.Tensor) -> np.ndarray:
    """Exact host copy: bf16 -> fp32 is exact; fp32 and ints unchanged."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def np64(t: torch.Tensor) -> np.ndarray:
    return np32(t).astype(np.float64)


def check_selection(S_gpu: np.ndarray, v_ref: np.ndarray, k: int, rel: float = 1e-5):
    """Selection parity for one row. Returns the number of undecided tokens."""
    N = v_ref.shape[0]
    k_eff = min(k, N)
    S_gpu = np.asarray(S_gpu)
    assert S_gpu.shape == (k,)
    sel = S_gpu[:k_eff]
    assert (S_gpu[k_eff:] == -1).all(), "padding must be -1"
    assert (sel >= 0).all() and (sel < N).all(), "index out of range"
    assert (np.diff(sel) > 0).all(), "indices must be strictly ascending"
    if k_eff == 0:
        return 0
    order = np.lexsort((np.arange(N), -v_ref))
    vk = v_ref[order[k_eff - 1]]
    vmax = v_ref.max()
    decided = np.abs(v_ref - vk) > rel * vmax
    in_ref = np.zeros(N, bool)
    in_ref[order[:k_eff]] = True
    in_gpu = np.zeros(N, bool)
    in_gpu[sel] = True
    bad = decided & (in_ref != in_gpu)
    assert not bad.any(), (
        f"{bad.sum()} decided tokens differ, e.g. {np.nonzero(bad)[0][:10]} "
        f"(v_ref={v_ref[bad][:5]}, k-th={vk}, vmax={vmax})")
    return int((~decided).sum())


def check_attention(out_gpu: np.ndarray, out_ref: np.ndarray, tol: float):
    """Per-head relative max error; returns the worst ratio err / (tol * max|ref|)."""
    err = np.abs(out_gpu - out_ref).max(axis=-1)
    scale = np.abs(out_ref).max(axis=-1)
    worst = 0.0
    for idx in np.ndindex(err.shape):
        if scale[idx] == 0:
            assert err[idx] == 0, f"head {idx}: expected zeros"
            continue
        r = err[idx] / (tol * scale[idx])
        worst = max(worst, r)
        assert r <= 1.0, f"head {idx}: err {err[idx]:.3e} > {tol} * {scale[idx]:.3e}"
    return worst


def rel_err(a: np.ndarray, b: np.ndarray) -> float:
    d = np.abs(a - b).max()
    s = np.abs(b).max()
    return float(d / s) if s > 0 else float(d)


def oracle_votes(q64: np.ndarray, K32: np.ndarray, n: int) -> np.ndarray:
    from oracle import ts_oracle as O
    return O.soft_vote(O.head_softmax(O.logits(q64, K32[:n])))


def check_run(ts, rc, mode: int, theta: float, sel_steps=None, att_steps=None, device="cuda"):
    """Runs rc.steps decode steps of a paged selection-cache run through the C ABI
    and checks them against the oracle. Every hit/miss decision is checked
    (except cosines within 1e-9 of theta); a hit must repeat the previous
    selection exactly. Selections of misses are checked at `sel_steps`, and
    attention outputs at `att_steps` (None: every step). The oracle's cache
    state follows the GPU's decisions and selections. Returns hits [T][B]."""
    import math
    import workloads as W
    from oracle import ts_oracle as O
    x = W.gen_run(rc, device=device)
    lens = x["seq_lens"].tolist()
    B = rc.batch
    cache = ts.SelCache(B, rc.num_q_heads, rc.head_dim, rc.k, mode=mode)
    pool_k, pool_v, pt = x["k_pool"], x["v_pool"], x["page_table"]
    hits, sels, outs = [], [], []
    for t in range(rc.steps):
        out, idx, hit = cache.decode_step(x["queries"][t], pool_k, pool_v, x["seq_lens"], theta,
                                          page_table=pt)
        hits.append(hit.clone())
        sels.append(idx.clone())
        outs.append(out.clone())
    torch.cuda.synchronize()
    h, m = cache.stats(B)
    cache.close()
    hits = torch.stack(hits).cpu().numpy()
    sels = torch.stack(sels).cpu().numpy()
    outs = torch.stack(outs).cpu().numpy().astype(np.float64)
    assert h == hits.sum(axis=0).tolist() and m == (rc.steps - hits.sum(axis=0)).tolist()
    kp, vp, ptn = np32(pool_k), np32(pool_v), pt.cpu().numpy()
    del pool_k, pool_v, x["k_pool"], x["v_pool"]
    Q = np64(x["queries"])
    sel_set = None if sel_steps is None else set(sel_steps)
    att_set = None if att_steps is None else set(att_steps)
    for b in range(B):
        # exact fp64 copies once per sequence (the oracle's dot products then
        # run on contiguous fp64 rows instead of upcasting on every call)
        Kb = O.paged_to_contiguous(kp, ptn[b], lens[b]).astype(np.float64)
        Vb = O.paged_to_contiguous(vp, ptn[b], lens[b]).astype(np.float64)
        ref_cache = O.SelectionCache(mode)
        for t in range(rc.steps):
            hit_ref, c = ref_cache.decide(Q[t, b], theta)
            if abs(c - theta) > 1e-9 or math.isnan(c):
                assert bool(hits[t, b]) == hit_ref, f"seq {b} step {t}: cos {c}"
            if hits[t, b]:
                assert np.array_equal(sels[t, b], sels[t - 1, b])
            elif sel_set is None or t in sel_set:
                check_selection(sels[t, b], oracle_votes(Q[t, b], Kb, lens[b]), rc.k)
            if att_set is None or t in att_set:
                ref = O.sparse_attention(Q[t, b], Kb, Vb, sels[t, b])
                check_attention(outs[t, b], ref, 1e-2)
            # advance the oracle state with the GPU's decision and selection
            if mode == 0 or not hits[t, b]:
                ref_cache.prev_q = Q[t, b].copy()
            ref_cache.prev_S = sels[t, b]
            ref_cache.valid = True
        del Kb, Vb
    return hits
