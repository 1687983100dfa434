"""The binding's host-side checks: every tensor the kernels index by batch row,
and every caller-provided output, is checked before anything is launched.

Each case hands one wrong tensor to an entry point and expects a ValueError
with no kernel launched (the library's per-kernel launch counters stay at 0).
The wrong tensors are never read by a kernel: the checks run first.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


def _case(B=2, Hq=8, Hkv=2, d=64, N=100, topk=16, dt=torch.bfloat16):
    dev = "cuda"
    return {
        "q": torch.zeros(B, Hq, d, dtype=dt, device=dev),
        "k": torch.zeros(B, N, Hkv, d, dtype=dt, device=dev),
        "v": torch.zeros(B, N, Hkv, d, dtype=dt, device=dev),
        "lens": torch.full((B,), N, dtype=torch.int32, device=dev),
        "idx": torch.zeros(B, topk, dtype=torch.int32, device=dev),
        "pool": torch.zeros(4 * B, 32, Hkv, d, dtype=dt, device=dev),
        "pt": torch.zeros(B, 4, dtype=torch.int32, device=dev),
        "B": B, "Hq": Hq, "Hkv": Hkv, "d": d, "N": N, "topk": topk,
    }


def _rejects(ts, fn):
    torch.cuda.synchronize()
    ts.profile_reset()
    ts.profile_enable(True)
    try:
        with pytest.raises(ValueError):
            fn()
    finally:
        ts.profile_enable(False)
    launched = {n: c for n, (c, _) in ts.profile_read().items() if c}
    assert not launched, f"kernels launched before the error: {launched}"


def _bad_decode_args(c):
    """(name, kwargs) pairs, each with one wrong tensor for a decode step."""
    B = c["B"]
    good = dict(q=c["q"], k_cache=c["k"], v_cache=c["v"], seq_lens=c["lens"])
    yield "k_cache_fewer_rows", {**good, "k_cache": c["k"][:B - 1], "v_cache": c["v"][:B - 1]}
    yield "v_cache_shape", {**good, "v_cache": c["v"][:, :50].contiguous()}
    yield "v_cache_dtype", {**good, "v_cache": c["v"].float()}
    yield "seq_lens_int64", {**good, "seq_lens": c["lens"].long()}
    yield "seq_lens_short", {**good, "seq_lens": c["lens"][:B - 1]}
    yield "page_table_int64", {**good, "k_cache": c["pool"], "v_cache": c["pool"],
                               "page_table": c["pt"].long()}
    yield "page_table_fewer_rows", {**good, "k_cache": c["pool"], "v_cache": c["pool"],
                                    "page_table": c["pt"][:B - 1]}


def test_decode_step_rejects(gpu_lib):
    ts = gpu_lib
    c = _case()
    cache = ts.SelCache(c["B"], c["Hq"], c["d"], c["topk"])
    for name, kw in _bad_decode_args(c):
        _rejects(ts, lambda: cache.decode_step(theta=0.9, **kw))
    good = dict(q=c["q"], k_cache=c["k"], v_cache=c["v"], seq_lens=c["lens"], theta=0.9)
    _rejects(ts, lambda: cache.decode_step(**good, out=torch.zeros(c["B"], c["Hq"], c["d"] + 1,
                                                                   device="cuda")))
    _rejects(ts, lambda: cache.decode_step(**good, idx_out=torch.zeros(c["B"], c["topk"] - 1,
                                                                       dtype=torch.int32,
                                                                       device="cuda")))
    _rejects(ts, lambda: cache.decode_step(**good, hit_out=torch.zeros(c["B"] - 1,
                                                                       dtype=torch.int32,
                                                                       device="cuda")))
    _rejects(ts, lambda: cache.reset(seq_mask=torch.ones(c["B"] - 1, dtype=torch.int32,
                                                         device="cuda")))
    _rejects(ts, lambda: cache.reset(seq_mask=torch.ones(c["B"], dtype=torch.int64,
                                                         device="cuda")))
    cache.close()


def test_score_attend_append_reject(gpu_lib):
    ts = gpu_lib
    c = _case()
    B = c["B"]
    for name, kw in _bad_decode_args(c):
        args = dict(kw)
        v = args.pop("v_cache")
        if name.startswith("v_cache"):
            _rejects(ts, lambda: ts.sparse_attend(v_cache=v, idx=c["idx"], **args))
            _rejects(ts, lambda: ts.dense_attend(v_cache=v, **args))
            continue
        _rejects(ts, lambda: ts.score(**args))
        _rejects(ts, lambda: ts.sparse_attend(v_cache=v, idx=c["idx"], **args))
        _rejects(ts, lambda: ts.dense_attend(v_cache=v, **args))
    good = dict(q=c["q"], k_cache=c["k"], v_cache=c["v"], seq_lens=c["lens"])
    _rejects(ts, lambda: ts.sparse_attend(idx=c["idx"][:B - 1], **good))
    _rejects(ts, lambda: ts.sparse_attend(idx=c["idx"].long(), **good))
    _rejects(ts, lambda: ts.score(c["q"], c["k"], c["lens"],
                                  votes=torch.zeros(B, c["N"] - 1, device="cuda")))
    kn = torch.zeros(B, c["Hkv"], c["d"], dtype=c["q"].dtype, device="cuda")
    _rejects(ts, lambda: ts.append_kv(kn, kn, c["k"][:B - 1], c["v"][:B - 1], c["lens"]))
    _rejects(ts, lambda: ts.append_kv(kn, kn, c["k"], c["v"], c["lens"].long()))
    _rejects(ts, lambda: ts.append_kv(kn, kn, c["pool"], c["pool"], c["lens"],
                                      page_table=c["pt"][:B - 1]))
    votes = torch.zeros(B, c["N"], device="cuda")
    _rejects(ts, lambda: ts.topk(votes, c["lens"][:B - 1], 4))
    _rejects(ts, lambda: ts.topk(votes, c["lens"].long(), 4))
    _rejects(ts, lambda: ts.topk(votes, c["lens"], 4, idx=torch.zeros(B, 3, dtype=torch.int32,
                                                                      device="cuda")))


def test_prefill_and_quest_reject(gpu_lib):
    ts = gpu_lib
    q = torch.zeros(8, 8, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(64, 2, 128, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(7, 16, dtype=torch.int32, device="cuda")
    _rejects(ts, lambda: ts.sparse_attend_prefill(q, kc, kc, 56, idx))
    _rejects(ts, lambda: ts.sparse_attend_prefill(q, kc, kc[:32], 24,
                                                  torch.zeros(8, 16, dtype=torch.int32,
                                                              device="cuda")))
    _rejects(ts, lambda: ts.select_prefill(q, kc, 56, 16, idx=idx))
    c = _case()
    meta = torch.zeros(c["pool"].shape[0], c["Hkv"], 2, c["d"], dtype=c["q"].dtype, device="cuda")
    _rejects(ts, lambda: ts.quest_select(c["q"], c["pool"], meta, c["pt"][:1], c["lens"], 2))
    _rejects(ts, lambda: ts.quest_select(c["q"], c["pool"], meta, c["pt"], c["lens"].long(), 2))
    _rejects(ts, lambda: ts.quest_select(c["q"], c["pool"], meta[:1], c["pt"], c["lens"], 2))
    pidx = torch.zeros(c["B"], c["Hkv"], 2, dtype=torch.int32, device="cuda")
    _rejects(ts, lambda: ts.quest_attend(c["q"], c["pool"], c["pool"], c["pt"], c["lens"],
                                         pidx[:1]))
    _rejects(ts, lambda: ts.quest_meta(c["pool"], c["pt"].long(), c["lens"]))
