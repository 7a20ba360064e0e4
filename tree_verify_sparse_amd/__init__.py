"""Verification attention, top-k KV selection and sparse draft attention on MI355X.

Python binding of libsv.so (include/sv.h).  Every step runs in the library's
HIP kernels; this module only marshals torch tensors (device memory and the
current stream) into the C ABI.  Importing works without a GPU; calling
requires the built library and a gfx950 device, and there is no fallback.

    out, scores = verify_attn(q, kv, prefix_len, parent=None, score_rows=[0, N-1])
    idx, count  = topk_select(scores, prefix_len, k, k_max)
    draft_out   = sparse_draft_attn(q1, kv, idx, count)
    ck, cv      = compact_kv(kv, idx, count, cap)          # once per selection
    draft_out   = dense_draft_attn(q1, ck, cv, n_rows)     # per draft token
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import SvError, SV_F32, SV_BF16  # noqa: F401

__all__ = ["KVCache", "Workspace", "verify_attn", "topk_select", "sparse_draft_attn", "compact_kv",
           "dense_draft_attn", "verify_workspace_size", "topk_workspace_size", "sparse_workspace_size",
           "dense_draft_workspace_size", "build_tree", "accept_commit", "verify_attn_per_head",
           "sparse_draft_attn_per_head", "select_sink_window", "timing_events", "SvError", "lib",
           "validate_kv", "validate_tree", "validate_index", "ContractError", "verify_attn_noalloc",
           "verify_select", "verify_select_workspace_size"]


def lib() -> ctypes.CDLL:
    return _lib.load()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


# ---------------------------------------------------------------------------
# Argument checks.  The C ABI sees only pointers and sizes, so tensors that
# disagree with each other (a float32 query with a bfloat16 cache, a head dim
# other than the cache's, an output or index buffer of the wrong shape) would
# make the kernels read or write past an allocation.  Every entry point below
# checks its tensors against each other first, before any pointer is taken or
# anything is launched, and raises ValueError.

def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_i32(t: Optional[torch.Tensor], shape: tuple, name: str, dev) -> None:
    if t is None:
        return
    _need(t.dtype == torch.int32, f"{name} must be int32, got {t.dtype}")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _need(t.device == dev, f"{name} is on {t.device}, the call runs on {dev}")


def _check_like(t: Optional[torch.Tensor], shape: tuple, dtype, name: str, dev) -> None:
    if t is None:
        return
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _need(t.device == dev, f"{name} is on {t.device}, the call runs on {dev}")


def _check_kv(kv: "KVCache", dtype, D: int, Hq: int, dev) -> None:
    _need(kv.k.dim() == 3 and tuple(kv.k.shape) == tuple(kv.v.shape), "kv.k and kv.v must both be [num_slots][Hkv][D]")
    _need(kv.k.dtype == kv.v.dtype, f"kv.k ({kv.k.dtype}) and kv.v ({kv.v.dtype}) must share a dtype")
    _need(kv.k.dtype == dtype, f"query dtype {dtype} differs from the KV cache's {kv.k.dtype}")
    _need(kv.D == D, f"query head dim {D} differs from the KV cache's {kv.D}")
    _need(Hq % kv.Hkv == 0, f"{Hq} query heads are not a multiple of the cache's {kv.Hkv} KV heads")
    _need(kv.k.device == dev and kv.v.device == dev, f"the KV cache is on {kv.k.device}, the call runs on {dev}")
    if kv.page_table is not None:
        pt = kv.page_table
        _need(pt.dtype == torch.int32 and pt.dim() == 2, "kv.page_table must be int32 [B][max_pages]")
        _need(pt.device == dev, f"kv.page_table is on {pt.device}, the call runs on {dev}")


@dataclasses.dataclass
class KVCache:
    """K/V of one layer, token-major [num_slots][Hkv][D] each.

    Contiguous (page_table None): slot of (b, i) = b * seq_stride + i.
    Paged: slot = page_table[b][i // page_size] * page_size + i % page_size.
    """
    k: torch.Tensor
    v: torch.Tensor
    seq_stride: int = 0
    page_table: Optional[torch.Tensor] = None
    page_size: int = 1

    def c_struct(self) -> _lib.SvKvCache:
        if self.k.shape != self.v.shape or self.k.dim() != 3:
            raise ValueError("k and v must both be [num_slots][Hkv][D]")
        pt = self.page_table
        return _lib.SvKvCache(
            _ptr(self.k), _ptr(self.v), _ptr(pt) if pt is not None else None,
            int(self.page_size) if pt is not None else 1,
            int(pt.shape[1]) if pt is not None else 0,
            int(self.seq_stride), int(self.k.shape[0]))

    @property
    def Hkv(self) -> int:
        return int(self.k.shape[1])

    @property
    def D(self) -> int:
        return int(self.k.shape[2])


class Workspace:
    """Reusable device scratch buffer (grown on demand, never shrunk)."""

    def __init__(self, device=None):
        self.buf: Optional[torch.Tensor] = None
        self.device = device

    def get(self, nbytes: int, device) -> tuple[Optional[int], int]:
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf.data_ptr(), self.buf.numel()


_default_ws: dict = {}


def _ws(workspace: Optional[Workspace], key: str) -> Workspace:
    if workspace is not None:
        return workspace
    return _default_ws.setdefault(key, Workspace())


def verify_workspace_size(B, N, Hq, Hkv, D, P_max, dtype, is_tree, n_score_rows, page_size=0) -> int:
    return int(lib().sv_verify_workspace_size(B, N, Hq, Hkv, D, P_max, dtype, int(bool(is_tree)), n_score_rows,
                                              int(page_size)))


def sparse_workspace_size(B, Hq, Hkv, D, max_idx) -> int:
    return int(lib().sv_sparse_workspace_size(B, Hq, Hkv, D, max_idx))


def verify_attn(q: torch.Tensor, kv: KVCache, prefix_len: torch.Tensor, *, P_max: int,
                parent: Optional[torch.Tensor] = None, score_rows: Optional[Sequence[int]] = None,
                scale: float = 0.0, out: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                workspace: Optional[Workspace] = None):
    """sv_verify_attn: q [B][N][Hq][D] -> (out [B][N][Hq][D], scores fp32 [B][P_max] or None).

    ``score_rows``: verify nodes whose logits are summed into the scores
    (None or [] = no scores).  ``parent``: int32 [B][N] draft tree or None (chain).
    """
    _need(q.dim() == 4, "q must be [B][N][Hq][D]")
    B, N, Hq, D = (int(x) for x in q.shape)
    dev = q.device
    _check_kv(kv, q.dtype, D, Hq, dev)
    _check_i32(prefix_len, (B,), "prefix_len", dev)
    _check_i32(parent, (B, N), "parent", dev)
    _check_like(out, tuple(q.shape), q.dtype, "out", dev)
    _check_like(scores, (B, int(P_max)), torch.float32, "scores", dev)
    L = lib()
    rows = [int(r) for r in (score_rows or [])]
    if out is None:
        out = torch.empty_like(q)
    if rows and scores is None:
        scores = torch.empty((B, P_max), dtype=torch.float32, device=q.device)
    rows_arr = (ctypes.c_int32 * max(1, len(rows)))(*rows)
    dt = _dtype_code(q)
    nbytes = verify_workspace_size(B, N, Hq, kv.Hkv, D, P_max, dt, parent is not None, len(rows),
                                   kv.page_size if kv.page_table is not None else 0)
    wptr, wlen = _ws(workspace, "verify").get(nbytes, q.device)
    kvs = kv.c_struct()
    if _debug_checks():
        _raise_on(validate_kv(kv, prefix_len, P_max=P_max, N=N))
        if parent is not None:
            _raise_on(validate_tree(parent))
    _lib.check(L.sv_verify_attn(_ptr(q), dt, B, N, Hq, kv.Hkv, D, ctypes.byref(kvs), _ptr(prefix_len), P_max,
                                _ptr(parent), rows_arr, len(rows), float(scale), _ptr(out),
                                _ptr(scores) if rows else None, wptr, wlen, _stream(q.device)))
    return out, (scores if rows else None)


def verify_attn_noalloc(q: torch.Tensor, kv: KVCache, prefix_len: torch.Tensor, *, P_max: int,
                        parent: Optional[torch.Tensor] = None, score_rows: Optional[Sequence[int]] = None,
                        scale: float = 0.0, out: Optional[torch.Tensor] = None,
                        scores: Optional[torch.Tensor] = None):
    """sv_verify_attn_noalloc: verify_attn on the library's static scratch (no
    workspace; the caller still passes or gets out and scores)."""
    _need(q.dim() == 4, "q must be [B][N][Hq][D]")
    B, N, Hq, D = (int(x) for x in q.shape)
    dev = q.device
    _check_kv(kv, q.dtype, D, Hq, dev)
    _check_i32(prefix_len, (B,), "prefix_len", dev)
    _check_i32(parent, (B, N), "parent", dev)
    _check_like(out, tuple(q.shape), q.dtype, "out", dev)
    _check_like(scores, (B, int(P_max)), torch.float32, "scores", dev)
    L = lib()
    rows = [int(r) for r in (score_rows or [])]
    if out is None:
        out = torch.empty_like(q)
    if rows and scores is None:
        scores = torch.empty((B, P_max), dtype=torch.float32, device=dev)
    rows_arr = (ctypes.c_int32 * max(1, len(rows)))(*rows)
    kvs = kv.c_struct()
    _lib.check(L.sv_verify_attn_noalloc(_ptr(q), _dtype_code(q), B, N, Hq, kv.Hkv, D, ctypes.byref(kvs),
                                        _ptr(prefix_len), P_max, _ptr(parent), rows_arr, len(rows), float(scale),
                                        _ptr(out), _ptr(scores) if rows else None, _stream(dev)))
    return out, (scores if rows else None)


def verify_select_workspace_size(B, N, Hq, Hkv, D, P_max, dtype, is_tree, n_score_rows, page_size=0) -> int:
    return int(lib().sv_verify_select_workspace_size(B, N, Hq, Hkv, D, P_max, dtype, int(bool(is_tree)),
                                                     n_score_rows, int(page_size)))


def verify_select(q: torch.Tensor, kv: KVCache, prefix_len: torch.Tensor, k: torch.Tensor, k_max: int, *,
                  P_max: int, parent: Optional[torch.Tensor] = None, score_rows: Sequence[int] = (0,),
                  scale: float = 0.0, out: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                  idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                  workspace: Optional[Workspace] = None):
    """sv_verify_select: verify_attn then topk_select on its scores, fused.
    -> (out [B][N][Hq][D], scores fp32 [B][P_max], idx int32 [B][k_max], count int32 [B])."""
    _need(q.dim() == 4, "q must be [B][N][Hq][D]")
    B, N, Hq, D = (int(x) for x in q.shape)
    dev = q.device
    _check_kv(kv, q.dtype, D, Hq, dev)
    _check_i32(prefix_len, (B,), "prefix_len", dev)
    _check_i32(parent, (B, N), "parent", dev)
    _check_i32(k, (B,), "k", dev)
    _check_like(out, tuple(q.shape), q.dtype, "out", dev)
    _check_like(scores, (B, int(P_max)), torch.float32, "scores", dev)
    _check_i32(idx, (B, int(k_max)), "idx", dev)
    _check_i32(count, (B,), "count", dev)
    rows = [int(r) for r in score_rows]
    _need(len(rows) > 0, "verify_select needs at least one score row")
    L = lib()
    out = torch.empty_like(q) if out is None else out
    scores = torch.empty((B, P_max), dtype=torch.float32, device=dev) if scores is None else scores
    idx = torch.empty((B, k_max), dtype=torch.int32, device=dev) if idx is None else idx
    count = torch.empty((B,), dtype=torch.int32, device=dev) if count is None else count
    rows_arr = (ctypes.c_int32 * len(rows))(*rows)
    dt = _dtype_code(q)
    nbytes = verify_select_workspace_size(B, N, Hq, kv.Hkv, D, P_max, dt, parent is not None, len(rows),
                                          kv.page_size if kv.page_table is not None else 0)
    wptr, wlen = _ws(workspace, "verify_select").get(nbytes, dev)
    kvs = kv.c_struct()
    if _debug_checks():
        _raise_on(validate_kv(kv, prefix_len, P_max=P_max, N=N))
        if parent is not None:
            _raise_on(validate_tree(parent))
    _lib.check(L.sv_verify_select(_ptr(q), dt, B, N, Hq, kv.Hkv, D, ctypes.byref(kvs), _ptr(prefix_len), P_max,
                                  _ptr(parent), rows_arr, len(rows), float(scale), _ptr(k), int(k_max), _ptr(out),
                                  _ptr(scores), _ptr(idx), _ptr(count), wptr, wlen, _stream(dev)))
    return out, scores, idx, count


def topk_workspace_size(B, P_max) -> int:
    return int(lib().sv_topk_workspace_size(B, P_max))


def topk_select(scores: torch.Tensor, prefix_len: torch.Tensor, k: torch.Tensor, k_max: int,
                idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                workspace: Optional[Workspace] = None):
    """sv_topk_select: -> (idx int32 [B][k_max] ascending, -1 padded; count int32 [B])."""
    _need(scores.dim() == 2 and scores.dtype == torch.float32, "scores must be float32 [B][P_max]")
    B, P_max = (int(x) for x in scores.shape)
    dev = scores.device
    _check_i32(prefix_len, (B,), "prefix_len", dev)
    _check_i32(k, (B,), "k", dev)
    _check_i32(idx, (B, int(k_max)), "idx", dev)
    _check_i32(count, (B,), "count", dev)
    L = lib()
    if idx is None:
        idx = torch.empty((B, k_max), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty((B,), dtype=torch.int32, device=scores.device)
    wptr, wlen = _ws(workspace, "topk").get(topk_workspace_size(B, P_max), scores.device)
    _lib.check(L.sv_topk_select(_ptr(scores), B, P_max, _ptr(prefix_len), _ptr(k), k_max, _ptr(idx), _ptr(count),
                                wptr, wlen, _stream(scores.device)))
    return idx, count


def sparse_draft_attn(q: torch.Tensor, kv: KVCache, idx: torch.Tensor, n_idx: torch.Tensor, *,
                      max_idx: Optional[int] = None, scale: float = 0.0, out: Optional[torch.Tensor] = None,
                      workspace: Optional[Workspace] = None):
    """sv_sparse_draft_attn: q [B][Hq][D], idx int32 [B][stride] logical positions, n_idx int32 [B]."""
    _need(q.dim() == 3, "q must be [B][Hq][D]")
    B, Hq, D = (int(x) for x in q.shape)
    dev = q.device
    _check_kv(kv, q.dtype, D, Hq, dev)
    _need(idx.dim() == 2 and int(idx.shape[0]) == B, "idx must be int32 [B][stride]")
    stride = int(idx.shape[1])
    _check_i32(idx, (B, stride), "idx", dev)
    _check_i32(n_idx, (B,), "n_idx", dev)
    _check_like(out, tuple(q.shape), q.dtype, "out", dev)
    max_idx = stride if max_idx is None else int(max_idx)
    _need(0 <= max_idx <= stride, f"max_idx = {max_idx} must lie in [0, {stride}]")
    L = lib()
    if out is None:
        out = torch.empty_like(q)
    dt = _dtype_code(q)
    nbytes = sparse_workspace_size(B, Hq, kv.Hkv, D, max_idx)
    wptr, wlen = _ws(workspace, "sparse").get(nbytes, q.device)
    kvs = kv.c_struct()
    if _debug_checks():
        _raise_on(validate_index(kv, idx, n_idx, max_idx=max_idx))
    _lib.check(L.sv_sparse_draft_attn(_ptr(q), dt, B, Hq, kv.Hkv, D, ctypes.byref(kvs), _ptr(idx), stride,
                                      _ptr(n_idx), max_idx, float(scale), _ptr(out), wptr, wlen,
                                      _stream(q.device)))
    return out


def verify_attn_per_head(q: torch.Tensor, kv: KVCache, prefix_len: torch.Tensor, *, P_max: int,
                         parent: Optional[torch.Tensor] = None, score_rows: Sequence[int] = (0,),
                         scale: float = 0.0, out: Optional[torch.Tensor] = None,
                         head_scores: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None):
    """sv_verify_attn_per_head: -> (out [B][N][Hq][D], head_scores fp32 [B][Hkv][P_max])."""
    _need(q.dim() == 4, "q must be [B][N][Hq][D]")
    B, N, Hq, D = (int(x) for x in q.shape)
    dev = q.device
    _check_kv(kv, q.dtype, D, Hq, dev)
    _check_i32(prefix_len, (B,), "prefix_len", dev)
    _check_i32(parent, (B, N), "parent", dev)
    _check_like(out, tuple(q.shape), q.dtype, "out", dev)
    _check_like(head_scores, (B, kv.Hkv, int(P_max)), torch.float32, "head_scores", dev)
    L = lib()
    rows = [int(r) for r in score_rows]
    if out is None:
        out = torch.empty_like(q)
    if head_scores is None:
        head_scores = torch.empty((B, kv.Hkv, P_max), dtype=torch.float32, device=q.device)
    rows_arr = (ctypes.c_int32 * max(1, len(rows)))(*rows)
    dt = _dtype_code(q)
    nbytes = verify_workspace_size(B, N, Hq, kv.Hkv, D, P_max, dt, parent is not None, len(rows),
                                   kv.page_size if kv.page_table is not None else 0)
    wptr, wlen = _ws(workspace, "verify").get(nbytes, q.device)
    kvs = kv.c_struct()
    _lib.check(L.sv_verify_attn_per_head(_ptr(q), dt, B, N, Hq, kv.Hkv, D, ctypes.byref(kvs), _ptr(prefix_len),
                                         P_max, _ptr(parent), rows_arr, len(rows), float(scale), _ptr(out),
                                         _ptr(head_scores), wptr, wlen, _stream(q.device)))
    return out, head_scores


def sparse_draft_attn_per_head(q: torch.Tensor, kv: KVCache, idx: torch.Tensor, n_idx: torch.Tensor, *,
                               max_idx: Optional[int] = None, scale: float = 0.0,
                               out: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None):
    """sv_sparse_draft_attn_per_head: idx int32 [B][Hkv][stride], n_idx int32 [B][Hkv]."""
    _need(q.dim() == 3, "q must be [B][Hq][D]")
    B, Hq, D = (int(x) for x in q.shape)
    dev = q.device
    _check_kv(kv, q.dtype, D, Hq, dev)
    _need(idx.dim() == 3 and tuple(idx.shape[:2]) == (B, kv.Hkv), "idx must be int32 [B][Hkv][stride]")
    stride = int(idx.shape[2])
    _check_i32(idx, (B, kv.Hkv, stride), "idx", dev)
    _check_i32(n_idx, (B, kv.Hkv), "n_idx", dev)
    _check_like(out, tuple(q.shape), q.dtype, "out", dev)
    max_idx = stride if max_idx is None else int(max_idx)
    _need(0 <= max_idx <= stride, f"max_idx = {max_idx} must lie in [0, {stride}]")
    L = lib()
    if out is None:
        out = torch.empty_like(q)
    dt = _dtype_code(q)
    wptr, wlen = _ws(workspace, "sparse").get(sparse_workspace_size(B, Hq, kv.Hkv, D, max_idx), q.device)
    kvs = kv.c_struct()
    if _debug_checks():
        _raise_on(validate_index(kv, idx, n_idx, max_idx=max_idx))
    _lib.check(L.sv_sparse_draft_attn_per_head(_ptr(q), dt, B, Hq, kv.Hkv, D, ctypes.byref(kvs), _ptr(idx), stride,
                                               _ptr(n_idx), max_idx, float(scale), _ptr(out), wptr, wlen,
                                               _stream(q.device)))
    return out


def select_sink_window(prefix_len: torch.Tensor, P_max: int, sink: int, window: int, k_max: int):
    """sv_select_sink_window: -> (idx int32 [B][k_max], count int32 [B])."""
    _need(prefix_len.dim() == 1, "prefix_len must be int32 [B]")
    B = int(prefix_len.shape[0])
    _check_i32(prefix_len, (B,), "prefix_len", prefix_len.device)
    L = lib()
    idx = torch.empty((B, k_max), dtype=torch.int32, device=prefix_len.device)
    count = torch.empty((B,), dtype=torch.int32, device=prefix_len.device)
    _lib.check(L.sv_select_sink_window(B, int(P_max), _ptr(prefix_len), int(sink), int(window), int(k_max), _ptr(idx),
                                       _ptr(count), _stream(prefix_len.device)))
    return idx, count


def compact_kv(kv: KVCache, idx: torch.Tensor, n_idx: torch.Tensor, cap: int, *, max_idx: Optional[int] = None,
               ck: Optional[torch.Tensor] = None, cv: Optional[torch.Tensor] = None):
    """sv_compact_kv: the listed rows gathered into dense ck, cv [B][cap][Hkv][D]
    (rows past n_idx[b] are left as they were; new buffers start zeroed)."""
    _need(idx.dim() == 2, "idx must be int32 [B][stride]")
    B, stride = int(idx.shape[0]), int(idx.shape[1])
    dev = kv.k.device
    _check_kv(kv, kv.k.dtype, kv.D, kv.Hkv, dev)
    _check_i32(idx, (B, stride), "idx", dev)
    _check_i32(n_idx, (B,), "n_idx", dev)
    max_idx = stride if max_idx is None else int(max_idx)
    _need(0 <= max_idx <= stride, f"max_idx = {max_idx} must lie in [0, {stride}]")
    shape = (B, cap, kv.Hkv, kv.D)
    _check_like(ck, shape, kv.k.dtype, "ck", dev)
    _check_like(cv, shape, kv.k.dtype, "cv", dev)
    L = lib()
    if ck is None:
        ck = torch.zeros(shape, dtype=kv.k.dtype, device=kv.k.device)
    if cv is None:
        cv = torch.zeros(shape, dtype=kv.v.dtype, device=kv.v.device)
    if tuple(ck.shape) != shape or tuple(cv.shape) != shape:
        raise ValueError(f"ck and cv must be {shape}")
    kvs = kv.c_struct()
    _lib.check(L.sv_compact_kv(_dtype_code(kv.k), B, kv.Hkv, kv.D, ctypes.byref(kvs), _ptr(idx), stride,
                               _ptr(n_idx), max_idx, _ptr(ck), _ptr(cv), int(cap), _stream(kv.k.device)))
    return ck, cv


def dense_draft_workspace_size(B, Hq, Hkv, D, cap, dtype) -> int:
    return int(lib().sv_dense_draft_workspace_size(B, Hq, Hkv, D, cap, dtype))


def dense_draft_attn(q: torch.Tensor, ck: torch.Tensor, cv: torch.Tensor, n_rows: torch.Tensor, *,
                     scale: float = 0.0, out: Optional[torch.Tensor] = None,
                     workspace: Optional[Workspace] = None):
    """sv_dense_draft_attn: q [B][Hq][D] over rows [0, n_rows[b]) of ck, cv [B][cap][Hkv][D]."""
    _need(q.dim() == 3, "q must be [B][Hq][D]")
    B, Hq, D = (int(x) for x in q.shape)
    if ck.dim() != 4 or ck.shape != cv.shape or int(ck.shape[0]) != B or int(ck.shape[3]) != D:
        raise ValueError("ck and cv must both be [B][cap][Hkv][D]")
    cap, Hkv = int(ck.shape[1]), int(ck.shape[2])
    dev = q.device
    _need(ck.dtype == q.dtype and cv.dtype == q.dtype, f"ck / cv ({ck.dtype}, {cv.dtype}) must have q's dtype {q.dtype}")
    _need(Hq % Hkv == 0, f"{Hq} query heads are not a multiple of {Hkv} KV heads")
    _need(ck.device == dev and cv.device == dev, "ck and cv must be on q's device")
    _check_i32(n_rows, (B,), "n_rows", dev)
    _check_like(out, tuple(q.shape), q.dtype, "out", dev)
    L = lib()
    if out is None:
        out = torch.empty_like(q)
    dt = _dtype_code(q)
    wptr, wlen = _ws(workspace, "dense").get(dense_draft_workspace_size(B, Hq, Hkv, D, cap, dt), q.device)
    _lib.check(L.sv_dense_draft_attn(_ptr(q), dt, B, Hq, Hkv, D, _ptr(ck), _ptr(cv), cap, _ptr(n_rows),
                                     float(scale), _ptr(out), wptr, wlen, _stream(q.device)))
    return out


def build_tree(logprobs: torch.Tensor, n_nodes: int):
    """sv_build_tree: logprobs fp64 [B][max_depth + 1][n_cand] (rows sorted
    decreasing) -> (parent, depth, rank), int32 [B][n_nodes] each."""
    L = lib()
    if logprobs.dtype != torch.float64 or logprobs.dim() != 3:
        raise ValueError("logprobs must be float64 [B][max_depth + 1][n_cand]")
    B, md1, nc = (int(x) for x in logprobs.shape)
    dev = logprobs.device
    parent = torch.empty((B, n_nodes), dtype=torch.int32, device=dev)
    depth = torch.empty_like(parent)
    rank = torch.empty_like(parent)
    _lib.check(L.sv_build_tree(B, int(n_nodes), md1 - 1, nc, _ptr(logprobs), _ptr(parent), _ptr(depth), _ptr(rank),
                               _stream(dev)))
    return parent, depth, rank


def accept_commit(draft_tokens: torch.Tensor, target_tokens: torch.Tensor, *, parent: Optional[torch.Tensor] = None,
                  kv: Optional[KVCache] = None, prefix_len: Optional[torch.Tensor] = None, P_max: int = 0):
    """sv_accept_commit: greedy acceptance (and, with kv, the accepted branch's
    K/V moved in place behind the prefix).  Returns (path int32 [B][N],
    n_accepted int32 [B], bonus int32 [B], new_prefix_len int32 [B] or None)."""
    _need(draft_tokens.dim() == 2, "draft_tokens must be int32 [B][N]")
    B, N = (int(x) for x in draft_tokens.shape)
    dev = draft_tokens.device
    _check_i32(draft_tokens, (B, N), "draft_tokens", dev)
    _check_i32(target_tokens, (B, N), "target_tokens", dev)
    _check_i32(parent, (B, N), "parent", dev)
    _check_i32(prefix_len, (B,), "prefix_len", dev)
    if kv is not None:
        _check_kv(kv, kv.k.dtype, kv.D, kv.Hkv, dev)
    L = lib()
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    new_p = torch.empty((B,), dtype=torch.int32, device=dev) if prefix_len is not None else None
    kvs = kv.c_struct() if kv is not None else None
    dt = _dtype_code(kv.k) if kv is not None else SV_BF16
    _lib.check(L.sv_accept_commit(dt, B, N, kv.Hkv if kv is not None else 1, kv.D if kv is not None else 128,
                                  ctypes.byref(kvs) if kvs is not None else None, _ptr(prefix_len), int(P_max),
                                  _ptr(parent), _ptr(draft_tokens), _ptr(target_tokens), _ptr(path), _ptr(n_acc),
                                  _ptr(bonus), _ptr(new_p), _stream(dev)))
    return path, n_acc, bonus, new_p


class timing_events:
    """Context manager: record (start, stop) hipEvents around the main verify
    kernel of every sv_verify_attn call made inside it (on the call's stream)."""

    def __init__(self, start: "torch.cuda.Event", stop: "torch.cuda.Event"):
        for e in (start, stop):
            if e.cuda_event == 0:   # torch creates its events lazily
                e.record()
        self.start, self.stop = start, stop

    def __enter__(self):
        _lib.check(lib().sv_set_verify_timing_events(self.start.cuda_event, self.stop.cuda_event))
        return self

    def __exit__(self, *exc):
        _lib.check(lib().sv_set_verify_timing_events(None, None))
        return False


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


# ---------------------------------------------------------------------------
# Device-array contract checks (sv_validate_*).  Each returns the error record
# (code, b, i, value) as host ints after synchronising the stream; (0, 0, 0, 0)
# means every check passed.  With SV_DEBUG_CHECKS=1 in the environment,
# verify_attn and sparse_draft_attn run them first (except under graph
# capture) and raise ContractError.

_CONTRACT = {
    1: "prefix_len[{b}] = {v} lies outside [0, P_max]",
    2: "position {i} of sequence {b} maps to no KV slot (page entry {v})",
    3: "parent[{b}][{i}] = {v} is not a valid parent",
    4: "n_idx of list {b} = {v} lies outside [0, max_idx]",
    5: "entry {i} of index list {b} is position {v}, negative or mapped to no KV slot",
}


class ContractError(ValueError):
    """A device array violates the documented contract of an entry point."""


def _debug_checks() -> bool:
    # the checks synchronise, which a stream under graph capture does not allow:
    # captured calls are not checked
    return os.environ.get("SV_DEBUG_CHECKS", "") == "1" and not torch.cuda.is_current_stream_capturing()


def _raise_on(rec) -> None:
    code, b, i, v = rec
    if code:
        raise ContractError(_CONTRACT.get(code, "contract violation {c}").format(b=b, i=i, v=v, c=code))


def _err_record(dev: torch.device):
    return torch.empty((4,), dtype=torch.int32, device=dev)


def _read_record(err: torch.Tensor):
    torch.cuda.current_stream(err.device).synchronize()
    return tuple(int(x) for x in err.cpu().tolist())


def validate_kv(kv: KVCache, prefix_len: torch.Tensor, *, P_max: int, N: int = 0):
    """sv_validate_kv: prefix lengths in [0, P_max], positions [0, P_b + N) mapped to slots."""
    err = _err_record(prefix_len.device)
    kvs = kv.c_struct()
    B = int(prefix_len.shape[0])
    _lib.check(lib().sv_validate_kv(B, int(N), ctypes.byref(kvs), _ptr(prefix_len), int(P_max), _ptr(err),
                                    _stream(prefix_len.device)))
    return _read_record(err)


def validate_tree(parent: torch.Tensor):
    """sv_validate_tree: parent [B][N], root -1, every other parent in [0, i)."""
    err = _err_record(parent.device)
    B, N = (int(x) for x in parent.shape)
    _lib.check(lib().sv_validate_tree(B, N, _ptr(parent), _ptr(err), _stream(parent.device)))
    return _read_record(err)


def validate_index(kv: KVCache, idx: torch.Tensor, n_idx: torch.Tensor, *, max_idx: Optional[int] = None):
    """sv_validate_index: idx [B][stride] (or [B][Hkv][stride]), counts n_idx [B] (or [B][Hkv])."""
    err = _err_record(idx.device)
    kvs = kv.c_struct()
    B = int(idx.shape[0])
    per_seq = int(idx.shape[1]) if idx.dim() == 3 else 1
    stride = int(idx.shape[-1])
    max_idx = stride if max_idx is None else int(max_idx)
    _lib.check(lib().sv_validate_index(B, per_seq, ctypes.byref(kvs), _ptr(idx), stride, _ptr(n_idx), max_idx,
                                       _ptr(err), _stream(idx.device)))
    return _read_record(err)
