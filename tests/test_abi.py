"""The C-ABI library loads, exports every symbol include/ts.h declares, and its
host-side validation returns the documented codes before any HIP call (so
these run without a GPU)."""
import ctypes
import os
import re

import pytest

import sparse_kv_cache_ts_amd as ts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    try:
        return ts.load()
    except RuntimeError as e:
        pytest.fail(f"libts.so must be built before the tests run: {e}")


def _header_functions():
    text = open(os.path.join(ROOT, "include", "ts.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ts_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header():
    lib = _lib()
    names = _header_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert sorted(ts.EXPORTS) == names


def test_version_and_strings():
    lib = _lib()
    assert lib.ts_abi_version() == 1
    for st in range(5):
        assert lib.ts_status_string(st).decode().startswith("TS_")
    assert b"unknown" in lib.ts_status_string(99)


def _layout(Hq=28, Hkv=4, d=128, dtype=ts.TS_BF16, max_len=1024, ps=0, stride=0, scale=0.0):
    return ts.KvLayout(Hq, Hkv, d, dtype, scale, ps, max_len, stride)


def _ws_size(fn, *args):
    n = ctypes.c_size_t(0)
    st = fn(*args, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw, want", [
    (dict(Hq=28, Hkv=3), ts.TS_ERR_INVALID_ARG),     # Hkv does not divide Hq
    (dict(d=96), ts.TS_ERR_UNSUPPORTED),             # head_dim
    (dict(dtype=7), ts.TS_ERR_INVALID_ARG),          # unknown dtype
    (dict(max_len=0), ts.TS_ERR_INVALID_ARG),
    (dict(ps=12, stride=100), ts.TS_ERR_INVALID_ARG),  # page size not a power of two
    (dict(ps=16, stride=10), ts.TS_ERR_INVALID_ARG),   # page table too short for max_len
    (dict(Hq=128, Hkv=128), ts.TS_ERR_UNSUPPORTED),  # too many KV heads
    (dict(Hq=32, Hkv=32, dtype=ts.TS_F32), ts.TS_ERR_UNSUPPORTED),         # fp32 d=128: <= 16
    (dict(Hq=64, Hkv=64, d=64, dtype=ts.TS_F32), ts.TS_ERR_UNSUPPORTED),  # fp32 d=64: <= 32
    (dict(scale=float("inf")), ts.TS_ERR_INVALID_ARG),
])
def test_layout_validation(kw, want):
    lib = _lib()
    L = _layout(**kw)
    st, _ = _ws_size(lib.ts_score_workspace_size, ctypes.byref(L), 1)
    assert st == want
    assert lib.ts_last_error().decode() != ""


@pytest.mark.parametrize("kw", [dict(Hq=64, Hkv=64), dict(Hq=16, Hkv=16, dtype=ts.TS_F32),
                                dict(Hq=32, Hkv=32, d=64, dtype=ts.TS_F32)])
def test_layout_kv_head_limits_accepted(kw):
    lib = _lib()
    L = _layout(**kw)
    st, n = _ws_size(lib.ts_score_workspace_size, ctypes.byref(L), 1)
    assert st == 0 and n > 0


def test_workspace_sizes_positive_and_monotone():
    lib = _lib()
    L = _layout(max_len=131072)
    st, a = _ws_size(lib.ts_decode_step_workspace_size, ctypes.byref(L), 1, 2048)
    assert st == 0 and a > 0
    st, b = _ws_size(lib.ts_decode_step_workspace_size, ctypes.byref(L), 4, 2048)
    assert st == 0 and b > a
    st, c = _ws_size(lib.ts_score_workspace_size, ctypes.byref(L), 1)
    assert st == 0 and 0 < c < a
    st, t = _ws_size(lib.ts_topk_workspace_size, 512, 65536, 4096)
    assert st == 0 and t > 0
    st, _ = _ws_size(lib.ts_topk_workspace_size, 0, 65536, 4096)
    assert st == ts.TS_ERR_INVALID_ARG
    st, _ = _ws_size(lib.ts_topk_workspace_size, 4, 100, 0)
    assert st == ts.TS_ERR_INVALID_ARG
    st, _ = _ws_size(lib.ts_sparse_attend_workspace_size, ctypes.byref(L), 1, 0)
    assert st == ts.TS_ERR_INVALID_ARG


def test_null_and_workspace_errors_enqueue_nothing():
    lib = _lib()
    L = _layout()
    fake = ctypes.c_void_p(0x1000)       # never dereferenced: validation fails first
    # NULL tensor pointer
    st = lib.ts_score(ctypes.byref(L), 1, None, fake, None, fake, fake, fake, 1 << 30, None)
    assert st == ts.TS_ERR_INVALID_ARG
    # paged layout without page table
    Lp = _layout(ps=16, stride=64)
    st = lib.ts_score(ctypes.byref(Lp), 1, fake, fake, None, fake, fake, fake, 1 << 30, None)
    assert st == ts.TS_ERR_INVALID_ARG
    # workspace too small
    st = lib.ts_score(ctypes.byref(L), 1, fake, fake, None, fake, fake, fake, 16, None)
    assert st == ts.TS_ERR_WORKSPACE
    assert "workspace" in lib.ts_last_error().decode()
    # misaligned workspace
    st = lib.ts_score(ctypes.byref(L), 1, fake, fake, None, fake, fake,
                      ctypes.c_void_p(0x1004), 1 << 30, None)
    assert st == ts.TS_ERR_INVALID_ARG
    # top-k
    st = lib.ts_topk(1, 100, fake, None, 5, fake, fake, 1 << 30, None)
    assert st == ts.TS_ERR_INVALID_ARG
    st = lib.ts_topk(1, 100, fake, fake, 0, fake, fake, 1 << 30, None)
    assert st == ts.TS_ERR_INVALID_ARG
    # sparse attention
    st = lib.ts_sparse_attend(ctypes.byref(L), 1, fake, fake, None, None, fake, fake, 8, fake,
                              fake, 1 << 30, None)
    assert st == ts.TS_ERR_INVALID_ARG
    # append: NULL new rows, paged layout without page table
    st = lib.ts_append_kv(ctypes.byref(L), 1, None, fake, fake, fake, None, fake, None)
    assert st == ts.TS_ERR_INVALID_ARG
    st = lib.ts_append_kv(ctypes.byref(Lp), 1, fake, fake, fake, fake, None, fake, None)
    assert st == ts.TS_ERR_INVALID_ARG
    st = lib.ts_append_kv(ctypes.byref(L), 0, fake, fake, fake, fake, None, fake, None)
    assert st == ts.TS_ERR_INVALID_ARG
    # page selection: contiguous layout, more than 8 query heads per KV head, NULLs, k_pages
    n = ctypes.c_size_t()
    assert lib.ts_quest_select_workspace_size(ctypes.byref(L), 1, 16, ctypes.byref(n)) == \
        ts.TS_ERR_UNSUPPORTED
    Lg = _layout(Hq=36, Hkv=4, ps=16, stride=64)
    assert lib.ts_quest_select_workspace_size(ctypes.byref(Lg), 1, 16, ctypes.byref(n)) == \
        ts.TS_ERR_UNSUPPORTED
    assert lib.ts_quest_select_workspace_size(ctypes.byref(Lp), 1, 0, ctypes.byref(n)) == \
        ts.TS_ERR_INVALID_ARG
    assert lib.ts_quest_select_workspace_size(ctypes.byref(Lp), 2, 16, ctypes.byref(n)) == ts.TS_OK
    assert n.value > 0
    st = lib.ts_quest_meta(ctypes.byref(Lp), 1, fake, None, fake, 0, fake, None)
    assert st == ts.TS_ERR_INVALID_ARG
    st = lib.ts_quest_select(ctypes.byref(Lp), 1, fake, fake, fake, fake, 16, None, None, fake,
                             1 << 30, None)
    assert st == ts.TS_ERR_INVALID_ARG
    st = lib.ts_quest_attend(ctypes.byref(Lp), 1, fake, fake, fake, fake, fake, fake, 16, fake,
                             fake, 16, None)
    assert st == ts.TS_ERR_WORKSPACE
    # decode step without a cache
    st = lib.ts_decode_step(None, ctypes.byref(L), 1, fake, fake, fake, None, fake, 0.9, fake,
                            None, None, fake, 1 << 30, None)
    assert st == ts.TS_ERR_INVALID_ARG


def test_sel_cache_argument_errors():
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.ts_sel_cache_create(0, 28, 128, 2048, 0, ctypes.byref(h)) == ts.TS_ERR_INVALID_ARG
    assert lib.ts_sel_cache_create(1, 28, 128, 0, 0, ctypes.byref(h)) == ts.TS_ERR_INVALID_ARG
    assert lib.ts_sel_cache_create(1, 28, 128, 16, 2, ctypes.byref(h)) == ts.TS_ERR_INVALID_ARG
    assert lib.ts_sel_cache_create(1, 28, 128, 16, 0, None) == ts.TS_ERR_INVALID_ARG
    assert lib.ts_sel_cache_reset(None, None, None) == ts.TS_ERR_INVALID_ARG
    assert lib.ts_sel_cache_destroy(None) == ts.TS_OK
