"""The seeded generators build the inputs they claim to (CPU only)."""
import math
from dataclasses import replace

import numpy as np
import torch

import workloads as W


def test_decode_shapes_and_determinism():
    cfg = W.TINY
    a = W.gen_decode(cfg)
    b = W.gen_decode(cfg)
    assert a["q"].shape == (1, 4, 64) and a["q"].dtype == torch.float32
    assert a["k_cache"].shape == (1, 4096, 2, 64)
    assert a["v_cache"].shape == (1, 4096, 2, 64)
    assert torch.equal(a["k_cache"], b["k_cache"]) and torch.equal(a["q"], b["q"])
    pos = a["special"][0]
    assert len(pos) == 16 and len(set(pos.tolist())) == 16
    # planted keys are 4x copies of the group's first query head
    G = 2
    for kv in range(2):
        want = 4.0 * a["q"][0, kv * G]
        assert torch.allclose(a["k_cache"][0, pos, kv], want.expand(16, -1))


def test_heavy_keys():
    cfg = W.QWEN_32K
    x = W.gen_decode(cfg)
    assert x["q"].dtype == torch.bfloat16
    pos = x["special"][0]
    assert len(pos) == math.floor(0.01 * 32768) == 327
    kf = x["k_cache"][0, pos].float()                 # [327][4][128]
    norms = torch.linalg.vector_norm(kf, dim=-1)
    assert torch.allclose(norms, torch.full_like(norms, 3 * math.sqrt(128)), rtol=1e-2)
    qf = x["q"][0].float()
    for kv in range(4):
        cos = (kf[:, kv] @ qf[kv * 7]) / (norms[:, kv] * qf[kv * 7].norm())
        assert (cos > 0.999).all()


def test_bf16_rounding_is_nearest_even():
    x = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], dtype=torch.float32)
    y = x.to(torch.bfloat16).float()
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa -> 1.0
    assert y[0].item() == 1.0
    assert y[1].item() == 1.0 + 2 ** -6      # tie rounds up to even
    assert y[2].item() == 1.0


def test_paged_run_layout():
    cfg = W.RunConfig("small-run", steps=40, batch=3, num_q_heads=8, num_kv_heads=2,
                      head_dim=16, min_len=100, max_len=300, dtype="bf16", k=32, seed=9)
    x = W.gen_run(cfg)
    lens = x["seq_lens"].tolist()
    assert all(100 <= n <= 300 for n in lens)
    pt = x["page_table"]
    pages = [(n + 15) // 16 for n in lens]
    used = torch.cat([pt[b, :pages[b]] for b in range(3)])
    assert sorted(used.tolist()) == list(range(sum(pages)))      # a permutation of the pool
    for b in range(3):
        assert (pt[b, pages[b]:] == -1).all()
    assert x["k_pool"].shape == (sum(pages), 16, 2, 16)
    assert x["queries"].shape == (40, 3, 8, 16)
    norms = torch.linalg.vector_norm(x["queries"].float(), dim=-1)
    assert torch.allclose(norms, torch.full_like(norms, 4.0), rtol=1e-2)


def test_query_process_cosines():
    Q = W.gen_query_process(64, 2, 32, 128, seed=3).double()
    flat = Q.reshape(64, 2, -1)
    cos = (flat[1:] * flat[:-1]).sum(-1) / (flat[1:].norm(dim=-1) * flat[:-1].norm(dim=-1))
    for t in range(1, 64):
        c = cos[t - 1]
        if t % 32 == 0:
            assert (c.abs() < 0.1).all()
        else:
            assert ((c > 0.93) & (c < 0.97)).all()


def test_prefill_rope_positions():
    cfg = W.PrefillConfig("p", chunk=4, n_ctx=32, num_q_heads=4, num_kv_heads=2, head_dim=8,
                          dtype="bf16", k=8, seed=1)
    x = W.gen_prefill(cfg)
    assert x["q"].shape == (4, 4, 8) and x["k_cache"].shape == (32, 2, 8)
    assert x["q_pos0"] == 28
    # rotary is a rotation: it preserves each vector's norm
    g = torch.Generator().manual_seed(1)
    raw = torch.randn(4, 4, 8, generator=g)
    rot = W.rope_rotate_half(raw, torch.arange(28, 32), 10000.0)
    assert torch.allclose(raw.norm(dim=-1), rot.norm(dim=-1), rtol=1e-5)
    # position 0 is the identity
    z = W.rope_rotate_half(raw[:1], torch.zeros(1), 10000.0)
    assert torch.allclose(z, raw[:1])


def test_gen_loop_layout():
    """The growing-cache loop: room for every step, pages mapped, zeros past each length."""
    cfg = replace(W.LOOP_RUN, batch=3, min_len=40, max_len=90, steps=7, page_size=16)
    for paged in (False, True):
        x = W.gen_loop(cfg, paged)
        y = W.gen_loop(cfg, paged)
        assert torch.equal(x["k_cache"], y["k_cache"]) and torch.equal(x["queries"], y["queries"])
        lens = x["seq_lens"].tolist()
        assert x["cap"] == max(lens) + cfg.steps
        assert x["k_new"].shape == (cfg.steps, cfg.batch, cfg.num_kv_heads, cfg.head_dim)
        if not paged:
            for b, n in enumerate(lens):
                assert (x["k_cache"][b, n:] == 0).all() and (x["k_cache"][b, n - 1] != 0).any()
            continue
        pt = x["page_table"]
        used = []
        for b, n in enumerate(lens):
            need = (n + cfg.steps + cfg.page_size - 1) // cfg.page_size
            assert (pt[b, :need] >= 0).all() and (pt[b, need:] == -1).all()
            used += pt[b, :need].tolist()
        assert sorted(used) == list(range(x["k_cache"].shape[0]))
