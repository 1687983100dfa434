"""TokenSelect decode-time hot path on MI355X: Python binding of libts.so.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in include/ts.h. PyTorch supplies device memory and the current
stream. If libts.so is missing the functions raise; there is no CPU fallback.

    import sparse_kv_cache_ts_amd as ts
    votes = ts.score(q, k_cache, seq_lens)                 # per-head soft votes
    idx = ts.topk(votes, seq_lens, k)                      # [B][k] ascending, -1 padded
    out = ts.sparse_attend(q, k_cache, v_cache, seq_lens, idx)
    cache = ts.SelCache(max_batch, Hq, d, k)
    out, idx, hit = cache.decode_step(q, k_cache, v_cache, seq_lens, theta=0.9)
    votes, idx = ts.select_prefill(q_chunk, k_ctx, q_pos0, k)
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "load", "lib_path", "TsError", "KvLayout", "make_layout", "score", "topk", "sparse_attend",
    "dense_attend", "sparse_attend_prefill", "append_kv", "quest_meta", "quest_select",
    "quest_attend",
    "SelCache", "score_prefill", "select_prefill", "Workspace", "EXPORTS",
    "profile_enable", "profile_reset", "profile_read",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None

TS_OK, TS_ERR_INVALID_ARG, TS_ERR_UNSUPPORTED, TS_ERR_WORKSPACE, TS_ERR_HIP = range(5)
NOALLOC_SCRATCH_BYTES = 32 << 20   # TS_NOALLOC_SCRATCH_BYTES of include/ts.h
TS_F32, TS_BF16 = 0, 1

# every symbol include/ts.h declares
EXPORTS = [
    "ts_abi_version", "ts_status_string", "ts_last_error",
    "ts_score_workspace_size", "ts_score",
    "ts_topk_workspace_size", "ts_topk",
    "ts_sparse_attend_workspace_size", "ts_sparse_attend",
    "ts_dense_attend_workspace_size", "ts_dense_attend",
    "ts_sparse_attend_prefill_workspace_size", "ts_sparse_attend_prefill",
    "ts_append_kv",
    "ts_quest_meta", "ts_quest_select_workspace_size", "ts_quest_select",
    "ts_quest_attend_workspace_size", "ts_quest_attend",
    "ts_sel_cache_create", "ts_sel_cache_reset", "ts_sel_cache_destroy", "ts_sel_cache_stats",
    "ts_decode_step_workspace_size", "ts_decode_step", "ts_decode_step_noalloc",
    "ts_score_prefill_workspace_size", "ts_score_prefill", "ts_select_prefill",
    "ts_profile_num_kernels", "ts_profile_kernel_name", "ts_profile_enable", "ts_profile_reset",
    "ts_profile_read",
]


class TsError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {detail}")


class KvLayout(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("page_size", ctypes.c_int32), ("max_len", ctypes.c_int32),
        ("page_table_stride", ctypes.c_int32),
    ]


def lib_path() -> str:
    """The in-tree library built from csrc/ (the only one this binding loads)."""
    return os.path.join(_PKG, "libts.so")


def load():
    """Load libts.so (built by `python -m sparse_kv_cache_ts_amd._build`)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m sparse_kv_cache_ts_amd._build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ, F32, F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float, ctypes.c_double
    L = ctypes.POINTER(KvLayout)
    SZP = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "ts_abi_version": ([], I32),
        "ts_status_string": ([I32], ctypes.c_char_p),
        "ts_last_error": ([], ctypes.c_char_p),
        "ts_score_workspace_size": ([L, I32, SZP], I32),
        "ts_score": ([L, I32, P, P, P, P, P, P, SZ, P], I32),
        "ts_topk_workspace_size": ([I32, I32, I32, SZP], I32),
        "ts_topk": ([I32, I32, P, P, I32, P, P, SZ, P], I32),
        "ts_sparse_attend_workspace_size": ([L, I32, I32, SZP], I32),
        "ts_sparse_attend": ([L, I32, P, P, P, P, P, P, I32, P, P, SZ, P], I32),
        "ts_dense_attend_workspace_size": ([L, I32, SZP], I32),
        "ts_dense_attend": ([L, I32, P, P, P, P, P, P, P, SZ, P], I32),
        "ts_sparse_attend_prefill_workspace_size": ([L, I32, I32, SZP], I32),
        "ts_sparse_attend_prefill": ([L, I32, I32, P, P, P, I32, P, I32, P, P, SZ, P], I32),
        "ts_append_kv": ([L, I32, P, P, P, P, P, P, P], I32),
        "ts_quest_meta": ([L, I32, P, P, P, I32, P, P], I32),
        "ts_quest_select_workspace_size": ([L, I32, I32, SZP], I32),
        "ts_quest_select": ([L, I32, P, P, P, P, I32, P, P, P, SZ, P], I32),
        "ts_quest_attend_workspace_size": ([L, I32, I32, SZP], I32),
        "ts_quest_attend": ([L, I32, P, P, P, P, P, P, I32, P, P, SZ, P], I32),
        "ts_sel_cache_create": ([I32, I32, I32, I32, I32, ctypes.POINTER(P)], I32),
        "ts_sel_cache_reset": ([P, P, P], I32),
        "ts_sel_cache_destroy": ([P], I32),
        "ts_sel_cache_stats": ([P, I32, P, P, P], I32),
        "ts_decode_step_workspace_size": ([L, I32, I32, SZP], I32),
        "ts_decode_step": ([P, L, I32, P, P, P, P, P, F64, P, P, P, P, SZ, P], I32),
        "ts_decode_step_noalloc": ([P, L, I32, P, P, P, P, P, F64, P, P, P, P], I32),
        "ts_score_prefill_workspace_size": ([L, I32, I32, I32, SZP], I32),
        "ts_score_prefill": ([L, I32, I32, P, P, I32, P, P, SZ, P], I32),
        "ts_select_prefill": ([L, I32, I32, P, P, I32, I32, P, P, P, SZ, P], I32),
        "ts_profile_num_kernels": ([], I32),
        "ts_profile_kernel_name": ([I32], ctypes.c_char_p),
        "ts_profile_enable": ([I32], I32),
        "ts_profile_reset": ([], I32),
        "ts_profile_read": ([I32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(F64)], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = lib
    return lib


def _check(st: int, where: str):
    if st != TS_OK:
        lib = load()
        raise TsError(st, where, lib.ts_last_error().decode())


# (every pointer argument is declared c_void_p, so plain integers pass as is)
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on(stream):
    """Allocation context of one call: its temporaries, default outputs and
    regrown workspaces are allocated on the stream its kernels run on, so the
    caching allocator hands that memory to no other stream while they may
    still use it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TS_BF16
    if t.dtype == torch.float32:
        return TS_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA (HIP) tensors")


# ---- host-side shape checks ---------------------------------------------------
# The kernels index every per-sequence tensor by the batch row (and the C ABI
# cannot see tensor extents), so each one is checked here before any launch:
# a tensor with fewer rows than the batch, or an int64 length/page table read
# as int32 pairs, would make the kernels read or write out of bounds.

def _rows(t: torch.Tensor, dim: int, n: int, name: str, dtype=None):
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != dim or t.shape[0] < n:
        raise ValueError(f"{name} must be {dim}-D with at least {n} rows (got {tuple(t.shape)})")


def _lens(t: torch.Tensor, n: int, name: str = "seq_lens"):
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() < n:
        raise ValueError(f"{name} must be a 1-D int32 tensor with at least {n} entries "
                         f"(got {t.dtype} {tuple(t.shape)})")


def _out(t: Optional[torch.Tensor], shape: tuple, dtype, name: str):
    """A caller-provided output: the given inner shape and dtype, >= shape[0] rows."""
    if t is None:
        return
    if (t.dtype != dtype or t.dim() != len(shape) or t.shape[0] < shape[0]
            or tuple(t.shape[1:]) != tuple(shape[1:])):
        raise ValueError(f"{name} must be {dtype} of shape {shape} (got {t.dtype} {tuple(t.shape)})")


def _kv(q, k_cache, v_cache, seq_lens, page_table):
    """q [B][Hq][d]; K (and V, same shape and dtype) contiguous with >= B rows
    or a pool with an int32 page table of >= B rows; int32 lengths >= B."""
    if q.dim() != 3:
        raise ValueError(f"q must be [batch][Hq][d] (got {tuple(q.shape)})")
    B = q.shape[0]
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache must be 4-D (got {tuple(k_cache.shape)})")
    if v_cache is not None and (v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype):
        raise ValueError("v_cache must have k_cache's shape and dtype")
    _lens(seq_lens, B)
    if page_table is None:
        if k_cache.shape[0] < B:
            raise ValueError(f"contiguous k_cache has {k_cache.shape[0]} rows for batch {B}")
    else:
        _rows(page_table, 2, B, "page_table", torch.int32)


def make_layout(q: torch.Tensor, k_cache: torch.Tensor, page_table: Optional[torch.Tensor] = None,
                scale: Optional[float] = None) -> KvLayout:
    """Layout from tensor shapes: q [B][Hq][d]; K contiguous [B][max_len][Hkv][d]
    or, with a page table [B][stride], a pool [P][page_size][Hkv][d]."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be 3-D and k_cache 4-D")
    B, Hq, d = q.shape
    if page_table is None:
        nb, max_len, Hkv, dk = k_cache.shape
        if nb < B:
            raise ValueError(f"contiguous k_cache has {nb} rows for batch {B}")
        ps, stride = 0, 0
    else:
        _, ps, Hkv, dk = k_cache.shape
        _rows(page_table, 2, B, "page_table", torch.int32)
        stride = page_table.shape[1]
        max_len = stride * ps
    if dk != d:
        raise ValueError("q and K head_dim differ")
    if k_cache.dtype != q.dtype:
        raise ValueError("q and K dtypes differ")
    return KvLayout(Hq, Hkv, d, _dtype_code(q), float(scale or 0.0), ps, max_len, stride)


class Workspace:
    """A reusable device scratch buffer (256-byte aligned by the allocator)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


def _ws(nbytes: int, device, ws: Optional[Workspace]):
    if ws is not None:
        return ws.get(nbytes, device)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def score(q, k_cache, seq_lens, page_table=None, scale=None, votes=None, ws=None, stream=None):
    """Per-head soft votes [B][max_len] fp32 (entries past seq_lens[b] unspecified)."""
    lib = load()
    _need_cuda(q, k_cache, seq_lens, page_table, votes)
    _kv(q, k_cache, None, seq_lens, page_table)
    L = make_layout(q, k_cache, page_table, scale)
    B = q.shape[0]
    _out(votes, (B, L.max_len), torch.float32, "votes")
    with _on(stream):
        if votes is None:
            votes = torch.empty(B, L.max_len, dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t()
        _check(lib.ts_score_workspace_size(ctypes.byref(L), B, ctypes.byref(n)),
               "ts_score_workspace_size")
        w = _ws(n.value, q.device, ws)
        _check(lib.ts_score(ctypes.byref(L), B, _ptr(q), _ptr(k_cache), _ptr(page_table),
                            _ptr(seq_lens), _ptr(votes), _ptr(w), w.numel(), _stream(stream)),
               "ts_score")
    return votes


def topk(votes, row_lens, k, idx=None, ws=None, stream=None):
    """Top-k of each row: [rows][k] int32, ascending, -1 padded, ties to the lower index."""
    lib = load()
    _need_cuda(votes, row_lens, idx)
    if votes.dtype != torch.float32 or votes.dim() != 2:
        raise ValueError("votes must be a 2-D fp32 tensor")
    rows, stride = votes.shape
    _lens(row_lens, rows, "row_lens")
    _out(idx, (rows, k), torch.int32, "idx")
    with _on(stream):
        if idx is None:
            idx = torch.empty(rows, k, dtype=torch.int32, device=votes.device)
        n = ctypes.c_size_t()
        _check(lib.ts_topk_workspace_size(rows, stride, k, ctypes.byref(n)), "ts_topk_workspace_size")
        w = _ws(n.value, votes.device, ws)
        _check(lib.ts_topk(rows, stride, _ptr(votes), _ptr(row_lens), k, _ptr(idx), _ptr(w),
                           w.numel(), _stream(stream)), "ts_topk")
    return idx


def sparse_attend(q, k_cache, v_cache, seq_lens, idx, page_table=None, scale=None, out=None,
                  ws=None, stream=None):
    """Attention of every query head over the rows idx names: [B][Hq][d] fp32."""
    lib = load()
    _need_cuda(q, k_cache, v_cache, seq_lens, idx, page_table, out)
    _kv(q, k_cache, v_cache, seq_lens, page_table)
    L = make_layout(q, k_cache, page_table, scale)
    B, Hq, d = q.shape
    _rows(idx, 2, B, "idx", torch.int32)
    k = idx.shape[1]
    _out(out, (B, Hq, d), torch.float32, "out")
    with _on(stream):
        if out is None:
            out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t()
        _check(lib.ts_sparse_attend_workspace_size(ctypes.byref(L), B, k, ctypes.byref(n)),
               "ts_sparse_attend_workspace_size")
        w = _ws(n.value, q.device, ws)
        _check(lib.ts_sparse_attend(ctypes.byref(L), B, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(page_table), _ptr(seq_lens), _ptr(idx), k, _ptr(out),
                                    _ptr(w), w.numel(), _stream(stream)), "ts_sparse_attend")
    return out


def dense_attend(q, k_cache, v_cache, seq_lens, page_table=None, scale=None, out=None, ws=None,
                 stream=None):
    """Full softmax attention over every cached token: [B][Hq][d] fp32."""
    lib = load()
    _need_cuda(q, k_cache, v_cache, seq_lens, page_table, out)
    _kv(q, k_cache, v_cache, seq_lens, page_table)
    L = make_layout(q, k_cache, page_table, scale)
    B, Hq, d = q.shape
    _out(out, (B, Hq, d), torch.float32, "out")
    with _on(stream):
        if out is None:
            out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t()
        _check(lib.ts_dense_attend_workspace_size(ctypes.byref(L), B, ctypes.byref(n)),
               "ts_dense_attend_workspace_size")
        w = _ws(n.value, q.device, ws)
        _check(lib.ts_dense_attend(ctypes.byref(L), B, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(page_table), _ptr(seq_lens), _ptr(out), _ptr(w), w.numel(),
                                   _stream(stream)), "ts_dense_attend")
    return out


class SelCache:
    """Selection-Cache state of up to max_batch sequences (device memory)."""

    def __init__(self, max_batch: int, num_q_heads: int, head_dim: int, k: int, mode: int = 0):
        self._lib = load()
        self.max_batch, self.num_q_heads, self.head_dim, self.k, self.mode = (
            max_batch, num_q_heads, head_dim, k, mode)
        h = ctypes.c_void_p()
        _check(self._lib.ts_sel_cache_create(max_batch, num_q_heads, head_dim, k, mode,
                                             ctypes.byref(h)), "ts_sel_cache_create")
        self._h = h
        self.ws = Workspace()
        # (layout, workspace bytes) per argument shape: both follow from the
        # shapes, dtypes and scale alone, so a decode loop builds them once
        self._plans = {}

    def close(self):
        if self._h is not None and self._h.value:
            _check(self._lib.ts_sel_cache_destroy(self._h), "ts_sel_cache_destroy")
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self, seq_mask=None, stream=None):
        """Reset every sequence (seq_mask None), or those with seq_mask[b] != 0
        (an int32 CUDA tensor, or a sequence of max_batch flags)."""
        if seq_mask is not None and not isinstance(seq_mask, torch.Tensor):
            flags = [1 if f else 0 for f in seq_mask]
            seq_mask = torch.tensor(flags, dtype=torch.int32, device="cuda")
        if seq_mask is not None:
            _need_cuda(seq_mask)
            _lens(seq_mask, self.max_batch, "seq_mask")
        _check(self._lib.ts_sel_cache_reset(self._h, _ptr(seq_mask), _stream(stream)),
               "ts_sel_cache_reset")

    def stats(self, n: Optional[int] = None, stream=None):
        n = self.max_batch if n is None else n
        hits = (ctypes.c_int64 * n)()
        misses = (ctypes.c_int64 * n)()
        _check(self._lib.ts_sel_cache_stats(self._h, n, hits, misses, _stream(stream)),
               "ts_sel_cache_stats")
        return list(hits), list(misses)

    def workspace_size(self, layout: KvLayout, batch: int) -> int:
        n = ctypes.c_size_t()
        _check(self._lib.ts_decode_step_workspace_size(ctypes.byref(layout), batch, self.k,
                                                       ctypes.byref(n)),
               "ts_decode_step_workspace_size")
        return n.value

    def _plan(self, q, k_cache, page_table, scale, sized: bool):
        key = (tuple(q.shape), q.dtype, tuple(k_cache.shape), k_cache.dtype,
               None if page_table is None else (tuple(page_table.shape), page_table.dtype), scale)
        plan = self._plans.get(key)
        if plan is None:
            L = make_layout(q, k_cache, page_table, scale)
            plan = (L, self.workspace_size(L, q.shape[0]) if sized else None)
            if len(self._plans) >= 64:
                self._plans.clear()
            self._plans[key] = plan
        elif sized and plan[1] is None:
            plan = (plan[0], self.workspace_size(plan[0], q.shape[0]))
            self._plans[key] = plan
        return plan

    def decode_step(self, q, k_cache, v_cache, seq_lens, theta: float, page_table=None, scale=None,
                    out=None, idx_out=None, hit_out=None, want_idx=True, stream=None):
        """One decode step: returns (out [B][Hq][d] fp32, idx [B][k] or None, hit [B] int32)."""
        _need_cuda(q, k_cache, v_cache, seq_lens, page_table, out, idx_out, hit_out)
        _kv(q, k_cache, v_cache, seq_lens, page_table)
        L, nbytes = self._plan(q, k_cache, page_table, scale, True)
        B = q.shape[0]
        _out(out, (B, self.num_q_heads, self.head_dim), torch.float32, "out")
        _out(idx_out, (B, self.k), torch.int32, "idx_out")
        _out(hit_out, (B,), torch.int32, "hit_out")
        dev = q.device
        with _on(stream):
            if out is None:
                out = torch.empty(B, self.num_q_heads, self.head_dim, dtype=torch.float32, device=dev)
            if idx_out is None and want_idx:
                idx_out = torch.empty(B, self.k, dtype=torch.int32, device=dev)
            if hit_out is None:
                hit_out = torch.empty(B, dtype=torch.int32, device=dev)
            w = self.ws.get(nbytes, dev)
            _check(self._lib.ts_decode_step(self._h, ctypes.byref(L), B, _ptr(q), _ptr(k_cache),
                                            _ptr(v_cache), _ptr(page_table), _ptr(seq_lens),
                                            float(theta), _ptr(out), _ptr(idx_out), _ptr(hit_out),
                                            _ptr(w), w.numel(), _stream(stream)), "ts_decode_step")
        return out, idx_out, hit_out

    def decode_step_noalloc(self, q, k_cache, v_cache, seq_lens, theta: float, out, hit_out,
                            idx_out=None, page_table=None, scale=None, stream=None):
        """The decode step on the library's static workspace (ts_decode_step_noalloc):
        no device memory is allocated by this call, so the caller passes every
        output (out [B][Hq][d] fp32, hit_out [B] int32, optional idx_out [B][k])."""
        _need_cuda(q, k_cache, v_cache, seq_lens, page_table, out, idx_out, hit_out)
        _kv(q, k_cache, v_cache, seq_lens, page_table)
        L = self._plan(q, k_cache, page_table, scale, False)[0]
        B = q.shape[0]
        if out is None or hit_out is None:
            raise ValueError("decode_step_noalloc needs caller-provided out and hit_out")
        _out(out, (B, self.num_q_heads, self.head_dim), torch.float32, "out")
        _out(idx_out, (B, self.k), torch.int32, "idx_out")
        _out(hit_out, (B,), torch.int32, "hit_out")
        _check(self._lib.ts_decode_step_noalloc(self._h, ctypes.byref(L), B, _ptr(q), _ptr(k_cache),
                                                _ptr(v_cache), _ptr(page_table), _ptr(seq_lens),
                                                float(theta), _ptr(out), _ptr(idx_out),
                                                _ptr(hit_out), _stream(stream)),
               "ts_decode_step_noalloc")
        return out, idx_out, hit_out


def _prefill_layout(q, k_ctx, scale):
    if q.dim() != 3 or k_ctx.dim() != 3:
        raise ValueError("q must be [chunk][Hq][d] and k_ctx [n_ctx][Hkv][d]")
    C, Hq, d = q.shape
    n_ctx, Hkv, dk = k_ctx.shape
    if dk != d or q.dtype != k_ctx.dtype:
        raise ValueError("q and K shapes/dtypes differ")
    return KvLayout(Hq, Hkv, d, _dtype_code(q), float(scale or 0.0), 0, n_ctx, 0)


def score_prefill(q, k_ctx, q_pos0: int, scale=None, votes=None, ws=None, stream=None):
    """Causal soft votes of a prefill chunk: [chunk][n_ctx] fp32 (zeros past q_pos0+i)."""
    lib = load()
    _need_cuda(q, k_ctx, votes)
    L = _prefill_layout(q, k_ctx, scale)
    C, n_ctx = q.shape[0], k_ctx.shape[0]
    _out(votes, (C, n_ctx), torch.float32, "votes")
    with _on(stream):
        if votes is None:
            votes = torch.empty(C, n_ctx, dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t()
        _check(lib.ts_score_prefill_workspace_size(ctypes.byref(L), C, n_ctx, 1, ctypes.byref(n)),
               "ts_score_prefill_workspace_size")
        w = _ws(n.value, q.device, ws)
        _check(lib.ts_score_prefill(ctypes.byref(L), C, q_pos0, _ptr(q), _ptr(k_ctx), n_ctx,
                                    _ptr(votes), _ptr(w), w.numel(), _stream(stream)),
               "ts_score_prefill")
    return votes


def select_prefill(q, k_ctx, q_pos0: int, k: int, scale=None, votes=None, idx=None, ws=None,
                   stream=None):
    """Soft votes and per-query top-k of a prefill chunk: (votes [C][n_ctx], idx [C][k])."""
    lib = load()
    _need_cuda(q, k_ctx, votes, idx)
    L = _prefill_layout(q, k_ctx, scale)
    C, n_ctx = q.shape[0], k_ctx.shape[0]
    _out(votes, (C, n_ctx), torch.float32, "votes")
    _out(idx, (C, k), torch.int32, "idx")
    with _on(stream):
        if votes is None:
            votes = torch.empty(C, n_ctx, dtype=torch.float32, device=q.device)
        if idx is None:
            idx = torch.empty(C, k, dtype=torch.int32, device=q.device)
        n = ctypes.c_size_t()
        _check(lib.ts_score_prefill_workspace_size(ctypes.byref(L), C, n_ctx, k, ctypes.byref(n)),
               "ts_score_prefill_workspace_size")
        w = _ws(n.value, q.device, ws)
        _check(lib.ts_select_prefill(ctypes.byref(L), C, q_pos0, _ptr(q), _ptr(k_ctx), n_ctx, k,
                                     _ptr(votes), _ptr(idx), _ptr(w), w.numel(), _stream(stream)),
               "ts_select_prefill")
    return votes, idx


def append_kv(k_new, v_new, k_cache, v_cache, seq_lens, page_table=None, stream=None):
    """Write each sequence's new K/V row at position seq_lens[b]; seq_lens += 1 (on device)."""
    lib = load()
    _need_cuda(k_new, v_new, k_cache, v_cache, seq_lens, page_table)
    if k_new.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("k_new must be [batch][Hkv][d] and the caches 4-D")
    B, Hkv, d = k_new.shape
    _lens(seq_lens, B)
    if v_new.shape != k_new.shape or k_new.dtype != k_cache.dtype or v_cache.shape != k_cache.shape \
            or v_new.dtype != k_new.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("new rows and caches disagree in shape or dtype")
    if page_table is None:
        if k_cache.shape[0] < B:
            raise ValueError(f"contiguous k_cache has {k_cache.shape[0]} rows for batch {B}")
        max_len, ps, stride = k_cache.shape[1], 0, 0
    else:
        _rows(page_table, 2, B, "page_table", torch.int32)
        ps, stride = k_cache.shape[1], page_table.shape[1]
        max_len = ps * stride
    if k_cache.shape[2:] != (Hkv, d):
        raise ValueError("new rows and caches disagree in heads or head_dim")
    L = KvLayout(Hkv, Hkv, d, _dtype_code(k_new), 0.0, ps, max_len, stride)
    _check(lib.ts_append_kv(ctypes.byref(L), B, _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                            _ptr(v_cache), _ptr(page_table), _ptr(seq_lens), _stream(stream)),
           "ts_append_kv")


def sparse_attend_prefill(q, k_ctx, v_ctx, q_pos0: int, idx, scale=None, out=None, ws=None,
                          stream=None):
    """Query i of a prefill chunk attends over its own selection idx[i]: [C][Hq][d] fp32."""
    lib = load()
    _need_cuda(q, k_ctx, v_ctx, idx, out)
    if v_ctx.shape != k_ctx.shape or v_ctx.dtype != k_ctx.dtype:
        raise ValueError("K and V shapes/dtypes differ")
    L = _prefill_layout(q, k_ctx, scale)
    C, Hq, d = q.shape
    _rows(idx, 2, C, "idx", torch.int32)
    n_ctx, k = k_ctx.shape[0], idx.shape[1]
    _out(out, (C, Hq, d), torch.float32, "out")
    with _on(stream):
        if out is None:
            out = torch.empty(C, Hq, d, dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t()
        _check(lib.ts_sparse_attend_prefill_workspace_size(ctypes.byref(L), C, k, ctypes.byref(n)),
               "ts_sparse_attend_prefill_workspace_size")
        w = _ws(n.value, q.device, ws)
        _check(lib.ts_sparse_attend_prefill(ctypes.byref(L), C, q_pos0, _ptr(q), _ptr(k_ctx),
                                            _ptr(v_ctx), n_ctx, _ptr(idx), k, _ptr(out), _ptr(w),
                                            w.numel(), _stream(stream)), "ts_sparse_attend_prefill")
    return out


def quest_meta(k_cache, page_table, seq_lens, meta=None, last_page_only=False, stream=None):
    """Per-page channel min/max keys: meta [P][Hkv][2][d] in the cache dtype (pool-page indexed)."""
    lib = load()
    _need_cuda(k_cache, page_table, seq_lens, meta)
    if k_cache.dim() != 4 or page_table.dim() != 2:
        raise ValueError("k_cache must be a pool [P][page][Hkv][d] and page_table 2-D")
    B = page_table.shape[0]
    _rows(page_table, 2, B, "page_table", torch.int32)
    _lens(seq_lens, B)
    P_, ps, Hkv, d = k_cache.shape
    with _on(stream):
        if meta is None:
            meta = torch.zeros(P_, Hkv, 2, d, dtype=k_cache.dtype, device=k_cache.device)
    if meta.shape != (P_, Hkv, 2, d) or meta.dtype != k_cache.dtype:
        raise ValueError("meta must be [pages][Hkv][2][d] in the cache dtype")
    L = KvLayout(Hkv, Hkv, d, _dtype_code(k_cache), 0.0, ps, ps * page_table.shape[1],
                 page_table.shape[1])
    _check(lib.ts_quest_meta(ctypes.byref(L), B, _ptr(k_cache), _ptr(page_table),
                             _ptr(seq_lens), 1 if last_page_only else 0, _ptr(meta),
                             _stream(stream)), "ts_quest_meta")
    return meta


def quest_select(q, k_cache, meta, page_table, seq_lens, k_pages: int, scale=None, scores=None,
                 page_idx=None, want_scores=False, ws=None, stream=None):
    """Top k_pages pages per (sequence, KV head): (page_idx [B][Hkv][k_pages], scores or None)."""
    lib = load()
    _need_cuda(q, k_cache, meta, page_table, seq_lens, scores, page_idx)
    if page_table is None:
        raise ValueError("page selection needs a page table")
    _kv(q, k_cache, None, seq_lens, page_table)
    L = make_layout(q, k_cache, page_table, scale)
    B = q.shape[0]
    P_, _, Hkv, d = k_cache.shape
    if meta.shape != (P_, Hkv, 2, d) or meta.dtype != k_cache.dtype:
        raise ValueError("meta must be [pages][Hkv][2][d] in the cache dtype")
    n_pages = -(-L.max_len // L.page_size)
    _out(page_idx, (B, Hkv, k_pages), torch.int32, "page_idx")
    _out(scores, (B, Hkv, n_pages), torch.float32, "scores")
    with _on(stream):
        if page_idx is None:
            page_idx = torch.empty(B, Hkv, k_pages, dtype=torch.int32, device=q.device)
        if scores is None and want_scores:
            scores = torch.empty(B, Hkv, n_pages, dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t()
        _check(lib.ts_quest_select_workspace_size(ctypes.byref(L), B, k_pages, ctypes.byref(n)),
               "ts_quest_select_workspace_size")
        w = _ws(n.value, q.device, ws)
        _check(lib.ts_quest_select(ctypes.byref(L), B, _ptr(q), _ptr(meta), _ptr(page_table),
                                   _ptr(seq_lens), k_pages, _ptr(scores), _ptr(page_idx), _ptr(w),
                                   w.numel(), _stream(stream)), "ts_quest_select")
    return page_idx, scores


def quest_attend(q, k_cache, v_cache, page_table, seq_lens, page_idx, scale=None, out=None,
                 ws=None, stream=None):
    """Each query head over the tokens of its KV head's pages: [B][Hq][d] fp32."""
    lib = load()
    _need_cuda(q, k_cache, v_cache, page_table, seq_lens, page_idx, out)
    if page_table is None:
        raise ValueError("page attention needs a page table")
    _kv(q, k_cache, v_cache, seq_lens, page_table)
    L = make_layout(q, k_cache, page_table, scale)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    if page_idx.dtype != torch.int32 or page_idx.dim() != 3 or page_idx.shape[0] < B \
            or page_idx.shape[1] != Hkv:
        raise ValueError("page_idx must be int32 [batch][Hkv][k_pages]")
    k_pages = page_idx.shape[2]
    _out(out, (B, Hq, d), torch.float32, "out")
    with _on(stream):
        if out is None:
            out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t()
        _check(lib.ts_quest_attend_workspace_size(ctypes.byref(L), B, k_pages, ctypes.byref(n)),
               "ts_quest_attend_workspace_size")
        w = _ws(n.value, q.device, ws)
        _check(lib.ts_quest_attend(ctypes.byref(L), B, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(page_table), _ptr(seq_lens), _ptr(page_idx), k_pages,
                                   _ptr(out), _ptr(w), w.numel(), _stream(stream)),
               "ts_quest_attend")
    return out


def profile_enable(on: bool = True):
    """Bracket every kernel launch with HIP events on its own stream (see ts.h)."""
    _check(load().ts_profile_enable(1 if on else 0), "ts_profile_enable")


def profile_reset():
    _check(load().ts_profile_reset(), "ts_profile_reset")


def profile_read() -> dict:
    """{kernel kind: (launches, total_ms)}; synchronizes the pending events."""
    lib = load()
    out = {}
    for i in range(lib.ts_profile_num_kernels()):
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        _check(lib.ts_profile_read(i, ctypes.byref(n), ctypes.byref(ms)), "ts_profile_read")
        out[lib.ts_profile_kernel_name(i).decode()] = (n.value, ms.value)
    return out
