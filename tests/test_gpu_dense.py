"""GPU parity of the dense (full) attention baseline against the fp64 oracle.

The oracle's attention over the selection 0 .. N-1 is full softmax attention
(pinned in test_oracle.py against torch's scaled_dot_product_attention).
Tolerance as for sparse attention: per (sequence, head) max-relative 1e-2 for
bf16, 1e-5 for fp32.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import ts_oracle as O
from tests.parity import check_attention, np32, np64

pytestmark = pytest.mark.gpu


def _cfg(name, B, Hq, Hkv, d, N, dtype, seed, max_len=None):
    return W.DecodeConfig(name, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, seq_len=N,
                          dtype=dtype, k=1, seed=seed, heavy_frac=0.01, max_len=max_len)


CASES = [
    _cfg("g2-d64-f32", 1, 4, 2, 64, 4096, "f32", 61),
    _cfg("g7-d128-bf16-ragged", 3, 28, 4, 128, 3001, "bf16", 62),
    _cfg("g4-d64-bf16", 2, 32, 8, 64, 777, "bf16", 63, max_len=1000),
    _cfg("g16-d64-bf16", 1, 16, 1, 64, 999, "bf16", 64),
    # head slices 3, 5 and 6 wide (G = 3, 5, 12)
    _cfg("g3-d128-bf16-ragged", 2, 6, 2, 128, 2500, "bf16", 65),
    _cfg("g5-d64-f32", 1, 20, 4, 64, 1500, "f32", 66),
    _cfg("g12-d128-bf16", 1, 24, 2, 128, 3333, "bf16", 67),
]


def _to_paged(K, V, lens, ps, seed):
    from tests.test_gpu_decode import _to_paged as tp
    return tp(K, V, lens, ps, seed)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_dense_attend(gpu_lib, cfg, paged):
    ts = gpu_lib
    x = W.gen_decode(cfg, device="cuda")
    lens = [cfg.seq_len - 501 * b for b in range(cfg.batch)]
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device="cuda")
    if paged:
        kp, vp, pt = _to_paged(x["k_cache"], x["v_cache"], lens, 16, 7)
        out = ts.dense_attend(x["q"], kp, vp, x["seq_lens"], page_table=pt)
    else:
        out = ts.dense_attend(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"])
    torch.cuda.synchronize()
    tol = 1e-5 if cfg.dtype == "f32" else 1e-2
    q64, o = np64(x["q"]), np64(out)
    for b, n in enumerate(lens):
        K, V = np32(x["k_cache"][b, :n]), np32(x["v_cache"][b, :n])
        ref = O.sparse_attention(q64[b], K, V, np.arange(n))
        check_attention(o[b], ref, tol)
        check_attention(o[b], ref, 2e-5)     # far inside the stated bound


def test_dense_attend_empty_and_one(gpu_lib):
    ts = gpu_lib
    cfg = _cfg("edge", 2, 8, 2, 64, 40, "bf16", 65)
    x = W.gen_decode(cfg, device="cuda")
    x["seq_lens"] = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    out = ts.dense_attend(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"])
    torch.cuda.synchronize()
    o = np64(out)
    assert (o[0] == 0).all()
    # one token: every head returns that token's value row of its KV head
    V = np32(x["v_cache"][1, 0])
    for h in range(8):
        np.testing.assert_allclose(o[1, h], V[h // 4], rtol=1e-6, atol=1e-6)


def test_dense_attend_full_size(gpu_lib):
    """Qwen2-7B shape, N = 131072: the baseline the sparse step is compared with."""
    ts = gpu_lib
    cfg = W.QWEN_128K
    x = W.gen_decode(cfg, device="cuda")
    out = ts.dense_attend(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"])
    torch.cuda.synchronize()
    n = cfg.seq_len
    ref = O.sparse_attention(np64(x["q"])[0], np32(x["k_cache"][0]), np32(x["v_cache"][0]),
                             np.arange(n))
    check_attention(np64(out)[0], ref, 1e-2)


def test_attend_more_columns_than_resident_groups(gpu_lib):
    """200 sequences x 4 KV heads = 800 (sequence, KV head) columns, more than
    the attention work-groups resident at once: the dense and the sparse plans
    grow their splits to whole lists (one split per column)."""
    ts = gpu_lib
    cfg = _cfg("g2-d64-bf16-b200", 200, 8, 4, 64, 300, "bf16", 65)
    x = W.gen_decode(cfg, device="cuda")
    lens = [1 + (37 * b) % cfg.seq_len for b in range(cfg.batch)]
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device="cuda")
    k = 128
    g = torch.Generator(device="cpu").manual_seed(66)
    idx = torch.full((cfg.batch, k), -1, dtype=torch.int32)
    for b, n in enumerate(lens):
        m = min(k, n)
        idx[b, :m] = torch.sort(torch.randperm(n, generator=g)[:m]).values.int()
    dense = ts.dense_attend(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"])
    sparse = ts.sparse_attend(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"], idx.cuda())
    torch.cuda.synchronize()
    q64, od, osp = np64(x["q"]), np64(dense), np64(sparse)
    for b in range(0, cfg.batch, 7):
        n = lens[b]
        K, V = np32(x["k_cache"][b, :n]), np32(x["v_cache"][b, :n])
        check_attention(od[b], O.sparse_attention(q64[b], K, V, np.arange(n)), 2e-5)
        check_attention(osp[b], O.sparse_attention(q64[b], K, V, idx[b].numpy()), 2e-5)
