"""Seeded synthetic inputs for the TokenSelect decode and prefill workloads.

This module only builds input tensors. It holds none of the method's
arithmetic (no scoring, softmax, voting, selection or attention), so both the
HIP path and the fp64 oracle can consume its output without sharing any of
the computation.

Every tensor comes from a ``torch.Generator`` seeded with the workload's
seed on the device the caller names. The same seed on a different device
gives different but equally distributed values, so a test always generates
once and hands the same bytes to both sides.

Workloads (attention shapes are those of the two models the TokenSelect
README evaluates, Qwen2-7B and Llama-3-8B; the pages give no token counts for
their pass-key run, so long contexts of 32K-256K stand in for it):

* ``TINY``        4 query / 2 KV heads, d=64, N=4096, fp32, k=256, 16 planted keys.
* ``QWEN_32K``    28/4 heads, d=128, N=32768, bf16, k=2048, 1% heavy keys.
* ``QWEN_128K``   the same shape and distribution at N=131072.
* ``LLAMA_4x128K`` 32/8 heads, d=128, 4 sequences of 131072, bf16, k=4096.
* ``PREFILL_64K`` 512-query chunk at the end of 65536 cached tokens, 32/8
  heads, d=128, bf16, rotary embedding applied at true positions, k=4096.
* ``SELCACHE_RUN`` 256 decode steps, 8 sequences of 16K-256K tokens, 32/8
  heads, d=128, bf16 paged KV (page size 16), k=4096, theta=0.9.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

__all__ = [
    "DecodeConfig", "PrefillConfig", "RunConfig",
    "TINY", "QWEN_32K", "QWEN_128K", "LLAMA_4x128K", "PREFILL_64K", "SELCACHE_RUN",
    "gen_decode", "gen_prefill", "gen_run", "gen_query_process", "rope_rotate_half",
    "torch_dtype",
]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclass(frozen=True)
class DecodeConfig:
    """One decode step for a batch of contiguous-KV sequences."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int            # tokens per sequence (all equal)
    dtype: str              # "f32" or "bf16": dtype of q, K and V
    k: int                  # top-k budget
    seed: int
    planted: int = 0        # keys that are scaled copies of the group's first query head
    planted_scale: float = 4.0
    heavy_frac: float = 0.0 # fraction of keys with 3x norm along the group's first query head
    heavy_norm: float = 3.0
    max_len: Optional[int] = None  # token capacity per sequence (>= seq_len)

    @property
    def capacity(self) -> int:
        return self.max_len if self.max_len is not None else self.seq_len


@dataclass(frozen=True)
class PrefillConfig:
    """Chunked-prefill selection: `chunk` queries at positions q_pos0 ... q_pos0+chunk-1."""
    name: str
    chunk: int
    n_ctx: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    k: int
    seed: int
    rope_base: float = 10000.0

    @property
    def q_pos0(self) -> int:
        # the chunk is the last `chunk` tokens of the cached context
        return self.n_ctx - self.chunk


@dataclass(frozen=True)
class RunConfig:
    """A run of consecutive decode steps over paged KV, for the selection cache."""
    name: str
    steps: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    min_len: int
    max_len: int
    dtype: str
    k: int
    seed: int
    page_size: int = 16
    theta: float = 0.9
    keep: float = 0.95      # weight of the previous query
    noise: float = 0.31     # weight of the fresh noise direction
    jump_every: int = 32    # a fresh random query every this many steps (t % jump_every == 0)
    heavy_frac: float = 0.01
    heavy_norm: float = 3.0


TINY = DecodeConfig("tiny-4q2kv-d64-4k-f32", batch=1, num_q_heads=4, num_kv_heads=2,
                    head_dim=64, seq_len=4096, dtype="f32", k=256, seed=0, planted=16)
QWEN_32K = DecodeConfig("qwen2-7b-shape-32k", batch=1, num_q_heads=28, num_kv_heads=4,
                        head_dim=128, seq_len=32768, dtype="bf16", k=2048, seed=1,
                        heavy_frac=0.01)
QWEN_128K = replace(QWEN_32K, name="qwen2-7b-shape-128k", seq_len=131072)
LLAMA_4x128K = DecodeConfig("llama3-8b-shape-4x128k", batch=4, num_q_heads=32, num_kv_heads=8,
                            head_dim=128, seq_len=131072, dtype="bf16", k=4096, seed=2,
                            heavy_frac=0.01)
PREFILL_64K = PrefillConfig("prefill-512x64k-llama3-8b-shape", chunk=512, n_ctx=65536,
                            num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                            k=4096, seed=3)
SELCACHE_RUN = RunConfig("selcache-run-8x256-paged", steps=256, batch=8, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, min_len=16384, max_len=262144,
                         dtype="bf16", k=4096, seed=4)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def _positions(n: int, count: int, g: torch.Generator, device) -> torch.Tensor:
    """`count` distinct positions in [0, n), uniformly without replacement, ascending."""
    if count <= 0:
        return torch.empty(0, dtype=torch.int64, device=device)
    perm = torch.randperm(n, generator=g, device=device)
    return torch.sort(perm[:count]).values


def gen_decode(cfg: DecodeConfig, device="cpu") -> dict:
    """Inputs of one decode step, contiguous KV.

    Returns q [B][Hq][d], k_cache / v_cache [B][capacity][Hkv][d] (cfg.dtype),
    seq_lens [B] int32, and `special` [B] lists of planted/heavy positions.
    Planted keys copy the group's first query head times `planted_scale`;
    heavy keys point along that head's direction with norm heavy_norm*sqrt(d).
    Slots past seq_len hold N(0,1) noise too (they must never be read).
    """
    B, Hq, Hkv, d = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    G = Hq // Hkv
    cap, N = cfg.capacity, cfg.seq_len
    g = _gen(cfg.seed, device)
    dt = torch_dtype(cfg.dtype)
    q = torch.randn(B, Hq, d, generator=g, device=device)
    K = torch.randn(B, cap, Hkv, d, generator=g, device=device)
    V = torch.randn(B, cap, Hkv, d, generator=g, device=device)
    q = q.to(dt)
    qf = q.float()
    special = []
    for b in range(B):
        pos_b = []
        if cfg.planted:
            pos = _positions(N, cfg.planted, g, device)
            for kv in range(Hkv):
                K[b, pos, kv, :] = cfg.planted_scale * qf[b, kv * G]
            pos_b.append(pos)
        if cfg.heavy_frac:
            n_heavy = int(math.floor(cfg.heavy_frac * N))
            pos = _positions(N, n_heavy, g, device)
            for kv in range(Hkv):
                K[b, pos, kv, :] = cfg.heavy_norm * math.sqrt(d) * _unit(qf[b, kv * G])
            pos_b.append(pos)
        special.append(torch.cat(pos_b) if pos_b else torch.empty(0, dtype=torch.int64, device=device))
    return {
        "q": q.contiguous(),
        "k_cache": K.to(dt).contiguous(),
        "v_cache": V.to(dt).contiguous(),
        "seq_lens": torch.full((B,), N, dtype=torch.int32, device=device),
        "special": special,
    }


def rope_rotate_half(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """Rotary position embedding in the rotate-half convention.

    x [..., n, H, d] float32, pos [n]: pairs (c, c+d/2) are rotated by the
    angle pos * base^(-2c/d). This shapes the synthetic data only.
    """
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-torch.arange(half, dtype=torch.float64, device=x.device) * 2.0 / d)
    ang = pos.to(torch.float64)[:, None] * inv[None, :]          # [n][half]
    cos = torch.cos(ang).float()[:, None, :]                      # [n][1][half]
    sin = torch.sin(ang).float()[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


def gen_prefill(cfg: PrefillConfig, device="cpu") -> dict:
    """Q [chunk][Hq][d] and K [n_ctx][Hkv][d], N(0,1) then rotary at true positions;
    V [n_ctx][Hkv][d] N(0,1) for the chunk's attention."""
    g = _gen(cfg.seed, device)
    dt = torch_dtype(cfg.dtype)
    Q = torch.randn(cfg.chunk, cfg.num_q_heads, cfg.head_dim, generator=g, device=device)
    K = torch.randn(cfg.n_ctx, cfg.num_kv_heads, cfg.head_dim, generator=g, device=device)
    qpos = torch.arange(cfg.q_pos0, cfg.q_pos0 + cfg.chunk, device=device)
    kpos = torch.arange(cfg.n_ctx, device=device)
    Q = rope_rotate_half(Q, qpos, cfg.rope_base)
    K = rope_rotate_half(K, kpos, cfg.rope_base)
    # V ~ N(0,1), drawn after Q and K so those do not depend on it
    V = torch.randn(cfg.n_ctx, cfg.num_kv_heads, cfg.head_dim, generator=g, device=device)
    return {"q": Q.to(dt).contiguous(), "k_cache": K.to(dt).contiguous(),
            "v_cache": V.to(dt).contiguous(), "q_pos0": cfg.q_pos0}


def gen_query_process(steps: int, batch: int, num_q_heads: int, head_dim: int, seed: int,
                      keep: float = 0.95, noise: float = 0.31, jump_every: int = 32,
                      device="cpu") -> torch.Tensor:
    """Queries [steps][B][Hq][d] float32 of a slowly drifting decode run.

    Per head: a fresh random unit direction at every t with t % jump_every == 0,
    else normalize(keep*q_{t-1} + noise*n_t) with n_t a random unit direction.
    Every head is then scaled to norm sqrt(d), so logits against N(0,1) keys
    are O(1). The recursion runs on unrounded float32 values.
    """
    g = _gen(seed, device)
    out = torch.empty(steps, batch, num_q_heads, head_dim, device=device)
    prev = None
    for t in range(steps):
        fresh = _unit(torch.randn(batch, num_q_heads, head_dim, generator=g, device=device))
        if prev is None or (jump_every > 0 and t % jump_every == 0):
            cur = fresh
        else:
            cur = _unit(keep * prev + noise * fresh)
        out[t] = cur
        prev = cur
    return out * math.sqrt(head_dim)


def gen_run(cfg: RunConfig, device="cpu", lens: Optional[list] = None) -> dict:
    """Paged KV plus the query process of a selection-cache decode run.

    Sequence lengths are uniform integers in [min_len, max_len] (or `lens`).
    The pool holds sum(ceil(N_b/page)) pages in a random order: page_table
    [B][max_pages] int32 maps each sequence's logical page to a pool page
    (unused entries are -1). Heavy keys of sequence b point along the first
    query head of each group at step 0.
    """
    g = _gen(cfg.seed, device)
    B, Hq, Hkv, d, P = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    G = Hq // Hkv
    dt = torch_dtype(cfg.dtype)
    if lens is None:
        lens = torch.randint(cfg.min_len, cfg.max_len + 1, (B,), generator=g, device=device).tolist()
    pages = [(n + P - 1) // P for n in lens]
    total = sum(pages)
    max_pages = max(pages) if pages else 0
    perm = torch.randperm(total, generator=g, device=device).to(torch.int32)
    page_table = torch.full((B, max(max_pages, 1)), -1, dtype=torch.int32, device=device)
    off = 0
    for b in range(B):
        page_table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    queries = gen_query_process(cfg.steps, B, Hq, d, cfg.seed + 1000, cfg.keep, cfg.noise,
                                cfg.jump_every, device=device)
    q_bf = queries.to(dt)
    # pool filled in slices to bound the float32 staging memory
    k_pool = torch.empty(max(total, 1), P, Hkv, d, dtype=dt, device=device)
    v_pool = torch.empty(max(total, 1), P, Hkv, d, dtype=dt, device=device)
    step = 4096
    for s in range(0, total, step):
        e = min(total, s + step)
        k_pool[s:e] = torch.randn(e - s, P, Hkv, d, generator=g, device=device).to(dt)
        v_pool[s:e] = torch.randn(e - s, P, Hkv, d, generator=g, device=device).to(dt)
    special = []
    q0 = q_bf[0].float()
    for b in range(B):
        n_heavy = int(math.floor(cfg.heavy_frac * lens[b]))
        pos = _positions(lens[b], n_heavy, g, device)
        pg = page_table[b, (pos // P)].long()
        slot = pos % P
        for kv in range(Hkv):
            vec = (cfg.heavy_norm * math.sqrt(d) * _unit(q0[b, kv * G])).to(dt)
            k_pool[pg, slot, kv, :] = vec
        special.append(pos)
    return {
        "queries": q_bf.contiguous(),          # [steps][B][Hq][d]
        "k_pool": k_pool, "v_pool": v_pool,    # [pages][P][Hkv][d]
        "page_table": page_table,              # [B][max_pages] int32
        "seq_lens": torch.tensor(lens, dtype=torch.int32, device=device),
        "special": special,
    }


LOOP_RUN = RunConfig("decode-loop-3x24-append", steps=24, batch=3, num_q_heads=16,
                     num_kv_heads=4, head_dim=128, min_len=900, max_len=5000, dtype="bf16",
                     k=256, seed=6, jump_every=8)


def gen_loop(cfg: RunConfig, paged: bool, device="cpu") -> dict:
    """A decode loop that grows the cache by one token per step.

    Initial lengths are uniform in [min_len, max_len]; the cache has room for
    steps more tokens per sequence. Contiguous: k_cache/v_cache
    [B][cap][Hkv][d] with cap = max(lens) + steps. Paged: a pool holding
    ceil((len_b + steps) / page) pages per sequence in a random order, and
    page_table [B][ceil(cap / page)] (unused entries -1). Keys, values and the
    per-step new rows k_new/v_new [steps][B][Hkv][d] are N(0,1); queries come
    from gen_query_process. Cache slots past each length hold zeros.
    """
    g = _gen(cfg.seed, device)
    B, Hq, Hkv, d, P, T = (cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                           cfg.page_size, cfg.steps)
    dt = torch_dtype(cfg.dtype)
    lens = torch.randint(cfg.min_len, cfg.max_len + 1, (B,), generator=g, device=device).tolist()
    cap = max(lens) + T
    k_new = torch.randn(T, B, Hkv, d, generator=g, device=device).to(dt)
    v_new = torch.randn(T, B, Hkv, d, generator=g, device=device).to(dt)
    queries = gen_query_process(T, B, Hq, d, cfg.seed + 1000, cfg.keep, cfg.noise,
                                cfg.jump_every, device=device).to(dt)
    out = {"queries": queries.contiguous(), "k_new": k_new, "v_new": v_new,
           "seq_lens": torch.tensor(lens, dtype=torch.int32, device=device), "cap": cap}
    if not paged:
        kc = torch.zeros(B, cap, Hkv, d, dtype=dt, device=device)
        vc = torch.zeros(B, cap, Hkv, d, dtype=dt, device=device)
        for b in range(B):
            kc[b, :lens[b]] = torch.randn(lens[b], Hkv, d, generator=g, device=device).to(dt)
            vc[b, :lens[b]] = torch.randn(lens[b], Hkv, d, generator=g, device=device).to(dt)
        out.update(k_cache=kc, v_cache=vc, page_table=None)
        return out
    pages = [(n + T + P - 1) // P for n in lens]
    total = sum(pages)
    perm = torch.randperm(total, generator=g, device=device).to(torch.int32)
    page_table = torch.full((B, (cap + P - 1) // P), -1, dtype=torch.int32, device=device)
    off = 0
    for b in range(B):
        page_table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    kp = torch.zeros(total, P, Hkv, d, dtype=dt, device=device)
    vp = torch.zeros(total, P, Hkv, d, dtype=dt, device=device)
    for b in range(B):
        n = lens[b]
        pos = torch.arange(n, device=device)
        pg = page_table[b, pos // P].long()
        kp[pg, pos % P] = torch.randn(n, Hkv, d, generator=g, device=device).to(dt)
        vp[pg, pos % P] = torch.randn(n, Hkv, d, generator=g, device=device).to(dt)
    out.update(k_cache=kp, v_cache=vp, page_table=page_table)
    return out
