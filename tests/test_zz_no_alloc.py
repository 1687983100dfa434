"""ts_decode_step_noalloc (the decode step on the library's static device
workspace, for callers that cannot allocate) against ts_decode_step with a
caller workspace: two calls in a row, the second on a smaller input, must give
bit-identical outputs, selections and decisions (the same kernels in the same
order). A step whose workspace exceeds the static array is refused on the
host with TS_ERR_WORKSPACE and launches nothing."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _inputs(B, N, seed):
    cfg = W.DecodeConfig(f"noalloc-b{B}-n{N}", batch=B, num_q_heads=28, num_kv_heads=4,
                         head_dim=128, seq_len=N, dtype="bf16", k=512, seed=seed, heavy_frac=0.01)
    return W.gen_decode(cfg, device="cuda")


def test_noalloc_matches_decode_step(gpu_lib):
    ts = gpu_lib
    ref = ts.SelCache(2, 28, 128, 512)
    noa = ts.SelCache(2, 28, 128, 512)
    # the larger call first, then a smaller one: the array keeps the first
    # call's intermediates, which the second must not depend on
    for B, N, seed, theta in ((2, 20000, 90, 0.9), (1, 3001, 91, 0.9)):
        x = _inputs(B, N, seed)
        args = (x["q"], x["k_cache"], x["v_cache"], x["seq_lens"], theta)
        o1, i1, h1 = ref.decode_step(*args)
        o2 = torch.full_like(o1, float("nan"))
        i2 = torch.full_like(i1, -7)
        h2 = torch.full_like(h1, -7)
        noa.decode_step_noalloc(*args, out=o2, hit_out=h2, idx_out=i2)
        torch.cuda.synchronize()
        assert torch.equal(h1, h2), (B, N)
        assert torch.equal(i1, i2), (B, N)
        assert torch.equal(o1, o2), (B, N)
        assert (h1 == 0).all()          # fresh state (first call) or fresh query: misses
    assert ref.stats(2) == noa.stats(2)
    ref.close()
    noa.close()


def test_noalloc_refuses_oversized_workspace(gpu_lib):
    ts = gpu_lib
    cache = ts.SelCache(2, 28, 128, 512)
    q = torch.zeros(2, 28, 128, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(4, 16, 4, 128, dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros(2, 16384, dtype=torch.int32, device="cuda")      # 262144 tokens per row
    lens = torch.zeros(2, dtype=torch.int32, device="cuda")
    lay = ts.make_layout(q, pool, pt)
    assert cache.workspace_size(lay, 2) > ts.NOALLOC_SCRATCH_BYTES
    out = torch.empty(2, 28, 128, device="cuda")
    hit = torch.empty(2, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    ts.profile_reset()
    ts.profile_enable(True)
    try:
        with pytest.raises(ts.TsError) as e:
            cache.decode_step_noalloc(q, pool, pool, lens, 0.9, out=out, hit_out=hit,
                                      page_table=pt)
    finally:
        ts.profile_enable(False)
    assert e.value.status == ts.TS_ERR_WORKSPACE
    assert not {n: c for n, (c, _) in ts.profile_read().items() if c}
    cache.close()
