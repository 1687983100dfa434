"""Decode steps on seeded random shapes against the fp64 oracle.

Sixteen combinations of batch (1-3, ragged lengths), KV heads (1-8), group
size (1, 2, 4, 7, 8), head_dim (64, 128), dtype (bf16, fp32), sequence
length (257 .. 20000), k (16 .. 5000) and cache layout (contiguous, or
paged with 1-, 16- or 64-token pages), drawn once from a fixed seed, plus
eight fixed shapes with group sizes 3, 5, 6, 10 and 12. Every sequence's
selection follows the decided-token rule and its attention is within the
dtype's tolerance of the oracle's over the GPU's selection.
"""
import random

import pytest
import torch

import workloads as W
from oracle import ts_oracle as O
from tests.parity import check_attention, check_selection, np32, np64
from tests.test_gpu_decode import _to_paged

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=2024):
    r = random.Random(seed)
    out = []
    for i in range(n):
        Hkv = r.choice([1, 2, 4, 8])
        G = r.choice([1, 2, 4, 7, 8])
        d = r.choice([64, 128])
        dt = r.choice(["bf16", "bf16", "f32"])
        if dt == "f32" and Hkv > (32 if d == 64 else 16):
            dt = "bf16"
        B = r.choice([1, 2, 3])
        N = r.choice([257, 1000, 4097, 20000])
        k = r.choice([16, 256, 1000, 2048, 5000])
        ps = r.choice([0, 0, 1, 16, 64])
        lens = [N] + [max(1, N - r.randrange(0, N)) for _ in range(B - 1)]
        out.append((i, B, Hkv * G, Hkv, d, dt, N, k, ps, lens))
    return out


# Query-head groups whose head slices take the 3-, 5- and 6-wide kernel
# instantiations (the slice is the largest divisor of G up to 8): G = 3, 5,
# 6, and G = 10, 12 as two slices of 5 and 6; bf16 and fp32, contiguous and
# paged, ragged batches, k above the length of a sequence.
ODD_GROUPS = [
    (100, 2, 6, 2, 128, "bf16", 3000, 200, 0, [3000, 1777]),
    (101, 1, 12, 4, 64, "f32", 2049, 300, 0, [2049]),
    (102, 1, 40, 8, 64, "bf16", 5000, 500, 16, [5000]),
    (103, 2, 5, 1, 128, "bf16", 777, 1000, 0, [777, 300]),
    (104, 1, 24, 4, 128, "f32", 2049, 300, 64, [2049]),
    (105, 1, 48, 8, 128, "bf16", 4097, 2048, 0, [4097]),
    (106, 3, 24, 2, 128, "bf16", 2000, 256, 1, [2000, 1999, 1]),
    (107, 1, 20, 2, 64, "bf16", 6000, 1024, 16, [6000]),
]


@pytest.mark.parametrize("case", ODD_GROUPS, ids=lambda c: f"c{c[0]}-h{c[2]}x{c[3]}-d{c[4]}-{c[5]}-n{c[6]}-k{c[7]}-p{c[8]}")
def test_decode_step_odd_groups(gpu_lib, case):
    test_decode_step_random_shape(gpu_lib, case)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"c{c[0]}-h{c[2]}x{c[3]}-d{c[4]}-{c[5]}-n{c[6]}-k{c[7]}-p{c[8]}")
def test_decode_step_random_shape(gpu_lib, case):
    ts = gpu_lib
    i, B, Hq, Hkv, d, dt, N, k, ps, lens = case
    cfg = W.DecodeConfig(f"rand{i}", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                         seq_len=N, dtype=dt, k=k, seed=3000 + i, heavy_frac=0.01)
    x = W.gen_decode(cfg, device="cuda")
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cache = ts.SelCache(B, Hq, d, k)
    if ps:
        kp, vp, pt = _to_paged(x["k_cache"], x["v_cache"], lens, ps, 4000 + i)
        out, idx, hit = cache.decode_step(x["q"], kp, vp, x["seq_lens"], 0.9, page_table=pt)
    else:
        out, idx, hit = cache.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"], 0.9)
    torch.cuda.synchronize()
    cache.close()
    q64, K32, V32 = np64(x["q"]), np32(x["k_cache"]), np32(x["v_cache"])
    gidx, o = idx.cpu().numpy(), np64(out)
    tol = 1e-5 if dt == "f32" else 1e-2
    for b, n in enumerate(lens):
        v = O.soft_vote(O.head_softmax(O.logits(q64[b], K32[b, :n])))
        check_selection(gidx[b], v, k)
        check_attention(o[b], O.sparse_attention(q64[b], K32[b, :n], V32[b, :n], gidx[b]), tol)
