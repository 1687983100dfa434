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
