"""GPU parity of the decode path (scoring, votes, top-k, sparse attention,
Selection Cache, decode step) against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ts_oracle as O
from tests.parity import check_attention, check_run, check_selection, np32, np64

pytestmark = pytest.mark.gpu

# vote tolerance: fp32 logits carry an absolute error of
# at most a few 1e-5 (base e) for logits of O(50); a vote is a sum of
# exp(s - lse) terms, so its relative error is bounded by about twice that.
VOTE_RTOL = 2e-4
VOTE_ATOL_REL_MAX = 1e-7


def _tol(dtype):
    return 1e-5 if dtype == torch.float32 else 1e-2


def _small_cfg(name, B, Hq, Hkv, d, N, dtype, k, seed, heavy=0.01, planted=0, max_len=None):
    return W.DecodeConfig(name, batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, seq_len=N,
                          dtype=dtype, k=k, seed=seed, heavy_frac=heavy, planted=planted,
                          max_len=max_len)


SMALL = [
    _small_cfg("g2-d64-f32", 1, 4, 2, 64, 4096, "f32", 256, 0, heavy=0, planted=16),
    _small_cfg("g1-d128-bf16", 2, 4, 4, 128, 3001, "bf16", 100, 11),
    _small_cfg("g7-d128-bf16", 1, 28, 4, 128, 5000, "bf16", 300, 12),
    _small_cfg("g4-d64-bf16", 2, 32, 8, 64, 2777, "bf16", 512, 13, max_len=3000),
    _small_cfg("g8-d128-f32", 1, 16, 2, 128, 1500, "f32", 64, 14),
    _small_cfg("g2-d128-bf16-ragged", 3, 4, 2, 128, 257, "bf16", 300, 15, heavy=0.05),
    _small_cfg("g16-d64-bf16", 1, 16, 1, 64, 999, "bf16", 77, 16),   # G > 8: two head slices
    _small_cfg("g2-d128-bf16-16kv", 2, 32, 16, 128, 1234, "bf16", 200, 17),  # 4 KV heads per wave
    _small_cfg("g3-d128-bf16-3kv", 2, 9, 3, 128, 700, "bf16", 50, 18),       # vector-ALU pass
    _small_cfg("g4-d128-bf16-1kv", 1, 4, 1, 128, 4500, "bf16", 300, 19),
]


def _oracle_votes(q64, K32, n):
    return O.soft_vote(O.head_softmax(O.logits(q64, K32[:n])))


def _varlen(x, lens):
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device=x["q"].device)
    return x


def _to_paged(K, V, lens, ps, seed):
    """Scatter contiguous [B][max_len][Hkv][d] caches into a shuffled page pool."""
    B, max_len, Hkv, d = K.shape
    g = torch.Generator(device="cpu").manual_seed(seed)
    pages = [(n + ps - 1) // ps for n in lens]
    total = sum(pages)
    perm = torch.randperm(total, generator=g).to(torch.int32)
    stride = (max_len + ps - 1) // ps
    pt = torch.full((B, stride), -1, dtype=torch.int32)
    kp = torch.zeros(total, ps, Hkv, d, dtype=K.dtype, device=K.device)
    vp = torch.zeros_like(kp)
    off = 0
    for b in range(B):
        pt[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
        for p in range(pages[b]):
            n = min(ps, lens[b] - p * ps)
            kp[pt[b, p].item(), :n] = K[b, p * ps:p * ps + n]
            vp[pt[b, p].item(), :n] = V[b, p * ps:p * ps + n]
    return kp, vp, pt.to(K.device)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_score_votes(gpu_lib, cfg):
    ts = gpu_lib
    x = W.gen_decode(cfg, device="cuda")
    lens = [cfg.seq_len - 37 * b for b in range(cfg.batch)]
    _varlen(x, lens)
    votes = ts.score(x["q"], x["k_cache"], x["seq_lens"])
    torch.cuda.synchronize()
    q64, K32 = np64(x["q"]), np32(x["k_cache"])
    for b, n in enumerate(lens):
        v = np64(votes[b, :n])
        ref = _oracle_votes(q64[b], K32[b], n)
        assert abs(v.sum() - cfg.num_q_heads) < 1e-4 * cfg.num_q_heads
        err = np.abs(v - ref)
        bound = VOTE_RTOL * ref + VOTE_ATOL_REL_MAX * ref.max()
        assert (err <= bound).all(), f"max rel err {(err / np.maximum(ref, 1e-30)).max():.3e}"


def test_score_votes_paged_matches_contiguous(gpu_lib):
    ts = gpu_lib
    cfg = _small_cfg("pg", 3, 16, 4, 128, 2000, "bf16", 128, 21, max_len=2048)
    x = W.gen_decode(cfg, device="cuda")
    lens = [2000, 700, 1]
    _varlen(x, lens)
    v_cont = ts.score(x["q"], x["k_cache"], x["seq_lens"])
    kp, vp, pt = _to_paged(x["k_cache"], x["v_cache"], lens, 16, 5)
    v_pag = ts.score(x["q"], kp, x["seq_lens"], page_table=pt)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        # same kernels, same arithmetic order: bit-identical
        assert torch.equal(v_cont[b, :n], v_pag[b, :n])


def _topk_rows(seed, stride=70010):
    g = torch.Generator(device="cpu").manual_seed(seed)
    lens = [0, 1, 5, 255, 4095, 4096, 4097, 10000, 70001]
    rows = []
    for i, n in enumerate(lens):
        kind = i % 5
        if kind == 4:
            # subnormals (down to 1e-45), +-0 and the smallest normals: the
            # selection compares floats, which must not flush subnormals
            r = torch.rand(stride, generator=g) * 2e-38
            r[::5] = -r[::5]
            r[::11] = 0.0
            r[1::11] = -0.0
        elif kind == 0:
            r = torch.rand(stride, generator=g)
        elif kind == 1:
            r = torch.randint(0, 4, (stride,), generator=g).float()        # heavy ties
        elif kind == 2:
            r = torch.randn(stride, generator=g)                             # negatives
            r[::7] = -0.0
            r[1::7] = 0.0
        else:
            r = torch.exp(torch.randn(stride, generator=g) * 8)              # wide range
        rows.append(r)
    return torch.stack(rows), lens


@pytest.mark.parametrize("k", [1, 7, 256, 4096, 5000])
def test_topk_exact(gpu_lib, k):
    ts = gpu_lib
    votes, lens = _topk_rows(k)
    vd = votes.cuda()
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx = ts.topk(vd, ld, k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    v = votes.numpy().astype(np.float64)
    for r, n in enumerate(lens):
        want = O.top_k(v[r, :n], k)
        assert np.array_equal(got[r], want), f"row {r} (len {n})"


@pytest.mark.parametrize("stride", [70012, 65533, 65536])
@pytest.mark.parametrize("k", [300, 9000])
def test_topk_exact_many_rows(gpu_lib, k, stride):
    """288 rows: the one-work-group-per-row kernel (16-byte loads when the row
    stride is a multiple of 4, single loads otherwise; rows of at most 65536
    keys build their histogram in the kernel)."""
    ts = gpu_lib
    parts = [_topk_rows(100 * k + i, stride) for i in range(32)]
    votes = torch.cat([p[0] for p in parts])
    lens = [min(n, stride) for n in sum((p[1] for p in parts), [])]
    vd = votes.cuda()
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx = ts.topk(vd, ld, k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    v = votes.numpy().astype(np.float64)
    for r, n in enumerate(lens):
        want = O.top_k(v[r, :n], k)
        assert np.array_equal(got[r], want), f"row {r} (len {n})"


def _crowded_row(seed, n, nb, ties):
    """n values whose k-th largest (k = 1500 + nb // 2) lies in one 10-bit
    second-level bin of its 12-bit first-level bin, with nb keys in that
    second-level bin (pairs of equal keys when `ties`)."""
    r = np.random.default_rng(seed)
    hi = r.uniform(2.0, 3.0, 1000).astype(np.float32)
    mid = r.uniform(1.01, 1.9, 500).astype(np.float32)         # same first-level bin, higher sub-bins
    nd = nb // 2 if ties else nb
    low10 = r.permutation(1024)[:nd].astype(np.uint32)
    sub = (np.uint32(0x3F800000) + low10).view(np.float32)      # 1.0 .. 1.0 + 1023 ulp
    if ties:
        sub = np.concatenate([sub, sub])
    low = r.uniform(0.0, 0.9, n - 1500 - sub.size).astype(np.float32)
    row = np.concatenate([hi, mid, sub, low])
    return row[r.permutation(n)], 1500 + nb // 2


@pytest.mark.parametrize("rows", [3, 256])
def test_topk_crowded_second_level_bin(gpu_lib, rows):
    """The k-th key's second-level bin holds at most 256 keys (ranked directly)
    or more (two further histogram passes), with and without equal keys: the
    partition/finalize kernels (3 rows) and the one-row-per-work-group kernel
    (256 rows)."""
    ts = gpu_lib
    n = 20000
    for nb in (1, 200, 256, 257, 600):
        for ties in (False, True):
            if ties and nb < 2:
                continue
            made = [_crowded_row(1000 * nb + 10 * i + ties, n, nb, ties) for i in range(rows)]
            k = made[0][1]
            votes = torch.from_numpy(np.stack([m[0] for m in made]))
            ld = torch.full((rows,), n, dtype=torch.int32, device="cuda")
            idx = ts.topk(votes.cuda(), ld, k)
            torch.cuda.synchronize()
            got = idx.cpu().numpy()
            v = votes.numpy().astype(np.float64)
            for r in range(rows):
                assert np.array_equal(got[r], O.top_k(v[r], k)), (nb, ties, r)


def test_topk_repeat_is_deterministic(gpu_lib):
    ts = gpu_lib
    votes, lens = _topk_rows(3)
    vd = votes.cuda()
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    a = ts.topk(vd, ld, 300).clone()
    b = ts.topk(vd, ld, 300)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


ATT = [
    ("f32-d64-g2", 2, 4, 2, 64, torch.float32, 3000, 256),
    ("f32-d128-g8", 1, 16, 2, 128, torch.float32, 1000, 100),
    ("bf16-d128-g7", 2, 28, 4, 128, torch.bfloat16, 5000, 2048),
    ("bf16-d64-g4", 3, 32, 8, 64, torch.bfloat16, 777, 300),
    ("bf16-d128-g16", 1, 16, 1, 128, torch.bfloat16, 600, 40),
]


@pytest.mark.parametrize("case", ATT, ids=lambda c: c[0])
@pytest.mark.parametrize("paged", [False, True])
def test_sparse_attend(gpu_lib, case, paged):
    ts = gpu_lib
    name, B, Hq, Hkv, d, dt, N, k = case
    g = torch.Generator(device="cpu").manual_seed(sum(map(ord, name)))
    q = torch.randn(B, Hq, d, generator=g).to(dt)
    K = torch.randn(B, N, Hkv, d, generator=g).to(dt)
    V = torch.randn(B, N, Hkv, d, generator=g).to(dt)
    lens = [N - 13 * b for b in range(B)]
    idx = torch.full((B, k), -1, dtype=torch.int32)
    for b in range(B):
        m = min(k, lens[b]) - b        # a few -1 slots in later rows
        sel = torch.randperm(lens[b], generator=g)[:m]
        idx[b, :m] = torch.sort(sel).values.int()
    qd, Kd, Vd = q.cuda(), K.cuda(), V.cuda()
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    if paged:
        Kd, Vd, pt = _to_paged(Kd, Vd, lens, 16, 7)
        out = ts.sparse_attend(qd, Kd, Vd, ld, idx.cuda(), page_table=pt)
    else:
        out = ts.sparse_attend(qd, Kd, Vd, ld, idx.cuda())
    torch.cuda.synchronize()
    o = np64(out)
    q64, K64, V64 = np64(q), np64(K), np64(V)
    ref = np.stack([O.sparse_attention(q64[b], K64[b, :lens[b]], V64[b, :lens[b]], idx[b].numpy())
                    for b in range(B)])
    check_attention(o, ref, _tol(dt))
    check_attention(o, ref, 2e-5)     # the kernel is far inside the stated bound


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_decode_step_miss(gpu_lib, cfg):
    ts = gpu_lib
    x = W.gen_decode(cfg, device="cuda")
    lens = [cfg.seq_len - 37 * b for b in range(cfg.batch)]
    _varlen(x, lens)
    cache = ts.SelCache(cfg.batch, cfg.num_q_heads, cfg.head_dim, cfg.k)
    out, idx, hit = cache.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"], 0.9)
    torch.cuda.synchronize()
    assert hit.cpu().tolist() == [0] * cfg.batch
    q64, K32, V32 = np64(x["q"]), np32(x["k_cache"]), np32(x["v_cache"])
    o = np64(out)
    gidx = idx.cpu().numpy()
    for b, n in enumerate(lens):
        v_ref = _oracle_votes(q64[b], K32[b], n)
        check_selection(gidx[b], v_ref, cfg.k)
        ref = O.sparse_attention(q64[b], K32[b, :n], V32[b, :n], gidx[b])
        check_attention(o[b], ref, _tol(x["q"].dtype))
        sp = x["special"][b].cpu().numpy()
        sp = sp[sp < n]
        if cfg.planted or cfg.heavy_frac:
            if len(sp) <= cfg.k:
                assert set(sp.tolist()) <= set(gidx[b].tolist())
    hits, misses = cache.stats(cfg.batch)
    assert hits == [0] * cfg.batch and misses == [1] * cfg.batch
    cache.close()


def test_decode_step_edge_cases(gpu_lib):
    """Empty sequence, k > N, and a one-token sequence in one batch."""
    ts = gpu_lib
    cfg = _small_cfg("edge", 3, 8, 2, 64, 50, "bf16", 64, 31, heavy=0)
    x = W.gen_decode(cfg, device="cuda")
    lens = [0, 50, 1]
    _varlen(x, lens)
    cache = ts.SelCache(3, 8, 64, 64)
    for step in range(2):
        out, idx, hit = cache.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"], 0.5)
        torch.cuda.synchronize()
        gidx = idx.cpu().numpy()
        assert (gidx[0] == -1).all() and (np32(out)[0] == 0).all()
        assert list(gidx[1][:50]) == list(range(50)) and (gidx[1][50:] == -1).all()
        assert gidx[2][0] == 0 and (gidx[2][1:] == -1).all()
        # step 0: all miss; step 1: same query -> hit, except the empty sequence
        assert hit.cpu().tolist() == ([0, 0, 0] if step == 0 else [0, 1, 1])
        q64, K32, V32 = np64(x["q"]), np32(x["k_cache"]), np32(x["v_cache"])
        for b in (1, 2):
            ref = O.sparse_attention(q64[b], K32[b, :lens[b]], V32[b, :lens[b]], gidx[b])
            check_attention(np64(out)[b], ref, 1e-2)


def test_selcache_run_mode0(gpu_lib):
    rc = W.RunConfig("small-run", steps=70, batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
                     min_len=300, max_len=3000, dtype="bf16", k=64, seed=41)
    hits = check_run(gpu_lib, rc, 0, 0.9)
    # drift (cos ~0.95) hits, the jumps at t % 32 == 0 miss
    for t in range(rc.steps):
        assert (hits[t] == (0 if t % 32 == 0 else 1)).all()


def test_selcache_run_mode1(gpu_lib):
    rc = W.RunConfig("small-run-anchor", steps=40, batch=2, num_q_heads=8, num_kv_heads=2,
                     head_dim=128, min_len=500, max_len=2000, dtype="bf16", k=100, seed=42)
    hits = check_run(gpu_lib, rc, 1, 0.9)
    assert 0 < hits.sum() < hits.size


def test_selcache_reset(gpu_lib):
    ts = gpu_lib
    cfg = _small_cfg("reset", 2, 8, 2, 64, 300, "bf16", 32, 51, heavy=0)
    x = W.gen_decode(cfg, device="cuda")
    cache = ts.SelCache(2, 8, 64, 32)
    args = (x["q"], x["k_cache"], x["v_cache"], x["seq_lens"], 0.5)
    _, _, h0 = cache.decode_step(*args)
    _, _, h1 = cache.decode_step(*args)
    cache.reset()
    _, _, h2 = cache.decode_step(*args)
    torch.cuda.synchronize()
    assert h0.tolist() == [0, 0] and h1.tolist() == [1, 1] and h2.tolist() == [0, 0]
    assert cache.stats(2) == ([0, 0], [1, 1])


def test_selcache_reset_one_sequence(gpu_lib):
    """A per-sequence reset in the middle of a run (a new sequence taking
    over batch slot 1): slot 1's next step misses, slots 0 and 2 keep
    hitting. Every decision matches the oracle's cache, whose state for slot
    1 alone is reset at the same step; hits repeat the previous selection,
    misses select what the oracle selects, and the counters restart."""
    ts = gpu_lib
    rc = W.RunConfig("reset-one-of-three", steps=12, batch=3, num_q_heads=8, num_kv_heads=2,
                     head_dim=128, min_len=600, max_len=1500, dtype="bf16", k=64, seed=43,
                     jump_every=0)
    x = W.gen_run(rc, device="cuda")
    B, t_reset = rc.batch, 6
    cache = ts.SelCache(B, rc.num_q_heads, rc.head_dim, rc.k)
    mask = torch.tensor([0, 1, 0], dtype=torch.int32, device="cuda")
    hits, sels = [], []
    for t in range(rc.steps):
        if t == t_reset:
            cache.reset(seq_mask=mask)
        _, idx, hit = cache.decode_step(x["queries"][t], x["k_pool"], x["v_pool"], x["seq_lens"],
                                        rc.theta, page_table=x["page_table"])
        hits.append(hit.clone())
        sels.append(idx.clone())
    torch.cuda.synchronize()
    hits = torch.stack(hits).cpu().numpy()
    sels = torch.stack(sels).cpu().numpy()
    expect = np.ones((rc.steps, B), dtype=np.int32)
    expect[0] = 0
    expect[t_reset, 1] = 0
    assert (hits == expect).all(), hits.T
    h, m = cache.stats(B)
    cache.close()
    assert h == [rc.steps - 1, rc.steps - t_reset - 1, rc.steps - 1] and m == [1, 1, 1]
    lens = x["seq_lens"].tolist()
    kp, ptn, Q = np32(x["k_pool"]), x["page_table"].cpu().numpy(), np64(x["queries"])
    for b in range(B):
        Kb = O.paged_to_contiguous(kp, ptn[b], lens[b])
        ref = O.SelectionCache(0)
        for t in range(rc.steps):
            if t == t_reset and b == 1:
                ref.reset()
            hit_ref, c = ref.decide(Q[t, b], rc.theta)
            assert bool(hits[t, b]) == hit_ref, f"seq {b} step {t}: cos {c}"
            if hits[t, b]:
                assert np.array_equal(sels[t, b], sels[t - 1, b])
            else:
                check_selection(sels[t, b], _oracle_votes(Q[t, b], Kb, lens[b]), rc.k)
            ref.prev_q, ref.prev_S, ref.valid = Q[t, b].copy(), sels[t, b], True


@pytest.mark.parametrize("n_copy", [5500, 11500], ids=["global-list", "row-rescan"])
def test_decode_step_crowded_threshold_bin(gpu_lib, n_copy):
    """Runs of identical keys give bitwise-equal votes, so the k-th vote's bin
    holds every copy: more candidates than the attention work-groups stage in
    LDS (5500: read from the global candidate list) or than the list keeps
    (11500: each work-group rescans the vote row). The selection is then the
    copies of lowest index (ties go to the lower index), exactly."""
    ts = gpu_lib
    Hq, Hkv, d, k = 8, 2, 64, 1000
    n = 500 + n_copy
    g = torch.Generator(device="cpu").manual_seed(97)
    q = torch.randn(1, Hq, d, generator=g)
    K = torch.randn(1, n, Hkv, d, generator=g)
    V = torch.randn(1, n, Hkv, d, generator=g)
    # the copies point along the mean query of each KV head's group: the
    # largest votes of the row
    for h in range(Hkv):
        dirn = q[0, h * (Hq // Hkv):(h + 1) * (Hq // Hkv)].mean(0)
        K[0, 500:, h] = 3.0 * dirn / dirn.norm() * d ** 0.5
    q, K, V = q.to(torch.bfloat16).cuda(), K.to(torch.bfloat16).cuda(), V.to(torch.bfloat16).cuda()
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    cache = ts.SelCache(1, Hq, d, k)
    out, idx, hit = cache.decode_step(q, K, V, lens, 0.9)
    torch.cuda.synchronize()
    assert hit.cpu().tolist() == [0]
    gidx = idx.cpu().numpy()[0]
    q64, K32, V32 = np64(q)[0], np32(K)[0], np32(V)[0]
    v_ref = _oracle_votes(q64, K32, n)
    assert np.array_equal(gidx, O.top_k(v_ref, k))
    assert np.array_equal(gidx, np.arange(500, 500 + k))
    check_attention(np64(out)[0], O.sparse_attention(q64, K32, V32, gidx), 1e-2)
    cache.close()


@pytest.mark.parametrize("ps", [1, 64, 512])
def test_decode_step_paged_page_sizes(gpu_lib, ps):
    """Paged decode steps with one-token pages, pages of 64 and pages larger
    than a scoring tile: the selection equals the contiguous cache's (the
    votes are the same bits) and the oracle's, the output matches the oracle."""
    ts = gpu_lib
    cfg = _small_cfg("paged-ps", 2, 8, 2, 128, 3000, "bf16", 256, 98, heavy=0.01)
    x = W.gen_decode(cfg, device="cuda")
    lens = [3000, 2111]
    _varlen(x, lens)
    c1 = ts.SelCache(2, 8, 128, 256)
    _, idx_c, _ = c1.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"], 0.9)
    kp, vp, pt = _to_paged(x["k_cache"], x["v_cache"], lens, ps, 99)
    c2 = ts.SelCache(2, 8, 128, 256)
    out, idx, hit = c2.decode_step(x["q"], kp, vp, x["seq_lens"], 0.9, page_table=pt)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_c)
    q64, K32, V32 = np64(x["q"]), np32(x["k_cache"]), np32(x["v_cache"])
    gidx, o = idx.cpu().numpy(), np64(out)
    for b, n in enumerate(lens):
        check_selection(gidx[b], _oracle_votes(q64[b], K32[b], n), 256)
        check_attention(o[b], O.sparse_attention(q64[b], K32[b, :n], V32[b, :n], gidx[b]), 1e-2)
    c1.close()
    c2.close()


@pytest.mark.parametrize("kind", ["tile-max-above-range", "every-term-below-range"])
def test_decode_step_logits_outside_fp64_sum_range(gpu_lib, kind):
    """A decode step sums each head's exp2 terms in fp64 (2^M per K-scan tile);
    when a tile's base-2 max exceeds 960, or when every term is below 2^-960,
    the vote kernel folds the tile partials instead. Both cases, then a normal
    step on the same cache (the sums and the flag must start it from zero),
    against the oracle's selection and attention."""
    ts = gpu_lib
    cfg = _small_cfg(kind, 1, 4, 2, 64, 3000, "bf16", 64, 41, heavy=0)
    x = W.gen_decode(cfg, device="cuda")
    K = x["k_cache"].float()
    q = x["q"].float()
    if kind == "tile-max-above-range":
        # 8 tokens whose key is 100 x the group's first query: base-2 logit
        # 100 * |q|^2 / 8 * log2(e), about 1150, for that head
        pos = torch.tensor([5, 700, 701, 1500, 2047, 2048, 2900, 2999], device="cuda")
        for kv in range(2):
            K[0, pos, kv, :] = 100.0 * q[0, 2 * kv]
    else:
        # every key points against both queries of its group: every logit is
        # near -1500 (base 2), the sum of 2^s underflows in fp64
        for kv in range(2):
            u = q[0, 2 * kv] + q[0, 2 * kv + 1]
            u = u / u.norm()
            K[0, :, kv, :] = -1500.0 * u + torch.randn(K.shape[1], 64, device="cuda")
    x["k_cache"] = K.to(torch.bfloat16).contiguous()
    cache = ts.SelCache(1, 4, 64, cfg.k)
    normal = W.gen_decode(_small_cfg("normal", 1, 4, 2, 64, 3000, "bf16", 64, 42), device="cuda")
    for step, xs in enumerate([x, normal]):
        out, idx, hit = cache.decode_step(xs["q"], xs["k_cache"], xs["v_cache"], xs["seq_lens"], 1.0)
        torch.cuda.synchronize()
        assert hit.cpu().tolist() == [0]
        q64, K32, V32 = np64(xs["q"]), np32(xs["k_cache"]), np32(xs["v_cache"])
        gidx = idx.cpu().numpy()
        check_selection(gidx[0], _oracle_votes(q64[0], K32[0], 3000), cfg.k)
        ref = O.sparse_attention(q64[0], K32[0, :3000], V32[0, :3000], gidx[0])
        check_attention(np64(out)[0], ref, 1e-2)
    cache.close()


def test_decode_step_fewer_votes_than_k_above_window(gpu_lib):
    """Every head's softmax sits on 8 planted keys (key = 200 x the head's own
    query, one query head per KV head): all other votes are exactly zero, so
    fewer than k keys fall in the partition's bin window [2112, 3136) and it
    reads all 4096 bins; the k-th vote is 0 and the zero votes tie."""
    ts = gpu_lib
    cfg = _small_cfg("fewer-than-k", 1, 2, 2, 64, 3000, "bf16", 64, 43, heavy=0)
    x = W.gen_decode(cfg, device="cuda")
    K = x["k_cache"].float()
    q = x["q"].float()
    pos = torch.tensor([3, 400, 401, 999, 1500, 2047, 2048, 2999], device="cuda")
    for kv in range(2):
        K[0, pos, kv, :] = 200.0 * q[0, kv]
    x["k_cache"] = K.to(torch.bfloat16).contiguous()
    cache = ts.SelCache(1, 2, 64, cfg.k)
    out, idx, hit = cache.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seq_lens"], 1.0)
    torch.cuda.synchronize()
    q64, K32, V32 = np64(x["q"]), np32(x["k_cache"]), np32(x["v_cache"])
    v_ref = _oracle_votes(q64[0], K32[0], 3000)
    assert (v_ref > 0).sum() == 8
    gidx = idx.cpu().numpy()
    check_selection(gidx[0], v_ref, cfg.k)
    assert set(pos.tolist()) <= set(gidx[0].tolist())
    ref = O.sparse_attention(q64[0], K32[0, :3000], V32[0, :3000], gidx[0])
    check_attention(np64(out)[0], ref, 1e-2)
    cache.close()
