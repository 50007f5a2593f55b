"""MI355X (gfx950) paged-KV attention step of one transformer layer.

Thin Python binding over libpagedkv.so (see include/pagedkv.h): it checks
tensor devices, dtypes and shapes, fills the C structs and calls the library
on the current HIP stream.  Every step of the computation runs in the
library's kernels; there is no other code path.

Names follow the mini-sglang Req/Batch model: cached_len, device_len,
extend_len = device_len - cached_len, table_idx, page_table (raw physical
rows, width a multiple of 32), out_loc, positions.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (PKV_STATUS_BAD_ALLOC, PKV_STATUS_BAD_DECODE, PKV_STATUS_BAD_LENGTHS, PKV_STATUS_BAD_OUT_LOC,
                   PKV_STATUS_BAD_PAGE_ROW, PKV_STATUS_BAD_POSITION, PKV_STATUS_BAD_TABLE_IDX,
                   PKV_STATUS_FREE_OVERFLOW, PKV_STATUS_OUT_OF_PAGES, PKV_STATUS_TOKEN_COUNT)

__all__ = ["PagedKVError", "KVPoolTensors", "KVCacheTensors", "BatchTensors", "MetadataBuffers", "kv_store", "build_attn_metadata",
           "build_attn_metadata_store",
           "paged_decode_attn", "paged_decode_attn_static", "paged_extend_attn", "plan_bytes", "workspace_bytes", "library_path", "plan_view",
           "rope_cos_sin_cache", "kv_store_rope", "PKV_STATUS_BAD_POSITION", "DecodeGraph", "PageFreeList",
           "BoundBatch", "BoundCall", "bind_kv_store", "bind_build_attn_metadata", "bind_build_attn_metadata_store",
           "bind_paged_decode_attn", "bind_paged_extend_attn",
           "PKV_STATUS_OUT_OF_PAGES", "PKV_STATUS_FREE_OVERFLOW",
           "PKV_STATUS_BAD_ALLOC", "PKV_STATUS_BAD_DECODE", "PKV_STATUS_BAD_LENGTHS", "PKV_STATUS_BAD_OUT_LOC",
           "PKV_STATUS_BAD_PAGE_ROW", "PKV_STATUS_BAD_TABLE_IDX", "PKV_STATUS_TOKEN_COUNT"]


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, code: int):
        msg = _lib.lib().pkv_error_string(code).decode()
        if code == _lib.PKV_ERR_HIP:
            msg += f" (hipError {_lib.lib().pkv_last_hip_error()})"
        super().__init__(f"{fn} failed: {msg}")
        self.code = code


def library_path() -> str:
    return _lib.LIB_PATH


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype, dims=None, contiguous: bool = True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got shape {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(fn: str, code: int):
    if code != _lib.PKV_OK:
        raise PagedKVError(fn, code)


@dataclass
class KVPoolTensors:
    """One layer's pool: k and v are bf16 [num_rows, Hkv, d] views whose rows
    may be further apart than Hkv * d elements (e.g. one layer of a pool that
    interleaves layers), with each row's heads contiguous."""
    k: torch.Tensor
    v: torch.Tensor
    page_size: int = 1

    def struct(self) -> _lib.KVPool:
        _need(self.k, "k_pool", torch.bfloat16, 3, contiguous=False)
        _need(self.v, "v_pool", torch.bfloat16, 3, contiguous=False)
        if self.k.shape != self.v.shape or self.k.stride() != self.v.stride():
            raise ValueError("k and v pools differ in shape or strides")
        n, hkv, d = self.k.shape
        if self.k.stride(2) != 1 or self.k.stride(1) != d:
            raise ValueError("each pool row's heads must be contiguous")
        return _lib.KVPool(self.k.data_ptr(), self.v.data_ptr(), n, self.k.stride(0), self.page_size, hkv, d, 0)


class KVCacheTensors:
    """All layers' K and V in one bf16 buffer, in the engine's layer-first
    ([2, L, N, Hkv, d]), page-first ([2, N, L, Hkv, d]) or row-interleaved
    ([N, L, 2, Hkv, d]: a row's K and V side by side) physical order; layer(i)
    is that layer's pool for the four calls."""

    LAYER_FIRST = _lib.PKV_LAYOUT_LAYER_FIRST
    PAGE_FIRST = _lib.PKV_LAYOUT_PAGE_FIRST
    ROW_INTERLEAVED = _lib.PKV_LAYOUT_ROW_INTERLEAVED

    def __init__(self, num_layers: int, num_rows: int, num_kv_heads: int, head_dim: int = 128, page_size: int = 1,
                 layout: int = _lib.PKV_LAYOUT_LAYER_FIRST, device="cuda"):
        shape = {self.LAYER_FIRST: (2, num_layers, num_rows, num_kv_heads, head_dim),
                 self.PAGE_FIRST: (2, num_rows, num_layers, num_kv_heads, head_dim),
                 self.ROW_INTERLEAVED: (num_rows, num_layers, 2, num_kv_heads, head_dim)}[layout]
        self.data = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        self.num_layers, self.num_rows, self.layout = num_layers, num_rows, layout
        self.num_kv_heads, self.head_dim, self.page_size = num_kv_heads, head_dim, page_size

    def struct(self) -> _lib.KVCache:
        return _lib.KVCache(self.data.data_ptr(), self.num_rows, self.num_layers, self.layout, self.page_size,
                            self.num_kv_heads, self.head_dim, 0)

    def layer_struct(self, layer_id: int) -> _lib.KVPool:
        """The library's description of one layer (base pointers, row stride)."""
        c, p = self.struct(), _lib.KVPool()
        _check("pkv_kv_cache_layer", _lib.lib().pkv_kv_cache_layer(ctypes.byref(c), layer_id, ctypes.byref(p)))
        return p

    def layer(self, layer_id: int) -> "KVPoolTensors":
        """Views of one layer's K and V rows; their struct() equals layer_struct()."""
        if self.layout == self.LAYER_FIRST:
            k, v = self.data[0, layer_id], self.data[1, layer_id]
        elif self.layout == self.PAGE_FIRST:
            k, v = self.data[0, :, layer_id], self.data[1, :, layer_id]
        else:
            k, v = self.data[:, layer_id, 0], self.data[:, layer_id, 1]
        pool = KVPoolTensors(k, v, self.page_size)
        want, got = self.layer_struct(layer_id), pool.struct()
        if (want.k, want.v, want.row_stride) != (got.k, got.v, got.row_stride):
            raise AssertionError("layer view and library layer description differ")
        return pool


@dataclass
class BatchTensors:
    """Per-request int32 device arrays and the batch's counts."""
    table_idx: torch.Tensor
    cached_len: torch.Tensor
    device_len: torch.Tensor
    num_decode: int
    num_tokens: int

    def struct(self) -> _lib.Batch:
        for name in ("table_idx", "cached_len", "device_len"):
            _need(getattr(self, name), name, torch.int32, 1)
        b = self.table_idx.numel()
        if self.cached_len.numel() != b or self.device_len.numel() != b:
            raise ValueError("table_idx, cached_len and device_len differ in length")
        return _lib.Batch(b, self.num_decode, self.num_tokens, self.table_idx.data_ptr(),
                          self.cached_len.data_ptr(), self.device_len.data_ptr())


@dataclass
class MetadataBuffers:
    """Caller-owned outputs of build_attn_metadata (fixed addresses)."""
    out_loc: torch.Tensor
    positions: torch.Tensor
    qo_indptr: torch.Tensor
    kv_indptr: torch.Tensor
    last_indices: torch.Tensor
    plan: torch.Tensor
    status: Optional[torch.Tensor] = None

    @classmethod
    def allocate(cls, max_reqs: int, max_tokens: int, num_qo_heads: int, num_kv_heads: int,
                 device="cuda") -> "MetadataBuffers":
        nbytes = plan_bytes(max_reqs, max_tokens, num_qo_heads, num_kv_heads)
        i32 = dict(dtype=torch.int32, device=device)
        return cls(out_loc=torch.zeros(max(max_tokens, 1), **i32), positions=torch.zeros(max(max_tokens, 1), **i32),
                   qo_indptr=torch.zeros(max_reqs + 1, **i32), kv_indptr=torch.zeros(max_reqs + 1, **i32),
                   last_indices=torch.zeros(max(max_reqs, 1), **i32),
                   plan=torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device),
                   status=torch.zeros(1, **i32))

    def struct(self) -> _lib.AttnMetadata:
        for name in ("out_loc", "positions", "qo_indptr", "kv_indptr", "last_indices"):
            _need(getattr(self, name), name, torch.int32, 1)
        _need(self.plan, "plan", torch.uint8, 1)
        if self.status is not None:
            _need(self.status, "status", torch.int32, 1)
        return _lib.AttnMetadata(self.out_loc.data_ptr(), self.positions.data_ptr(), self.qo_indptr.data_ptr(),
                                 self.kv_indptr.data_ptr(), self.last_indices.data_ptr(), self.plan.data_ptr(),
                                 self.plan.numel(), _ptr(self.status))


def plan_bytes(max_reqs: int, max_tokens: int, num_qo_heads: int, num_kv_heads: int) -> int:
    n = _lib.lib().pkv_plan_bytes(max_reqs, max_tokens, num_qo_heads, num_kv_heads)
    if n == 0:
        raise ValueError("invalid plan size query")
    return n


def plan_view(max_reqs: int, max_tokens: int, num_qo_heads: int, num_kv_heads: int) -> dict:
    """Where the plan of such a batch keeps its work lists (pkv_plan_view_layout)."""
    v = _lib.PlanView()
    _check("pkv_plan_view_layout", _lib.lib().pkv_plan_view_layout(max_reqs, max_tokens, num_qo_heads,
                                                                    num_kv_heads, ctypes.byref(v)))
    return {name: getattr(v, name) for name, _ in _lib.PlanView._fields_}


def workspace_bytes(max_reqs: int, num_qo_heads: int, head_dim: int = 128) -> int:
    n = _lib.lib().paged_attn_workspace_bytes(max_reqs, num_qo_heads, head_dim)
    if n == 0:
        raise ValueError("invalid workspace size query")
    return n


def _kv_store_args(pool, k_new, v_new, out_loc, status):
    p = pool.struct()
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    _need(out_loc, "out_loc", torch.int32, 1)
    t = k_new.shape[0]
    if v_new.shape != k_new.shape or k_new.shape[1:] != pool.k.shape[1:] or out_loc.numel() < t:
        raise ValueError("k_new / v_new / out_loc shapes do not match the pool")
    if status is not None:
        _need(status, "status", torch.int32, 1)
    return (ctypes.byref(p), k_new.data_ptr(), v_new.data_ptr(), out_loc.data_ptr(), t, _ptr(status)), (p,)


def kv_store(pool: KVPoolTensors, k_new: torch.Tensor, v_new: torch.Tensor, out_loc: torch.Tensor,
             status: Optional[torch.Tensor] = None, stream=None) -> None:
    args, _keep = _kv_store_args(pool, k_new, v_new, out_loc, status)
    _check("kv_store", _lib.lib().kv_store(*args, _stream(stream)))


def _metadata_args(batch, page_table, page_size, num_pool_rows, alloc_rows, num_qo_heads, num_kv_heads, meta):
    b = batch.struct()
    _need(page_table, "page_table", torch.int32, 2)
    _need(alloc_rows, "alloc_rows", torch.int32, 1)
    if meta.out_loc.numel() < batch.num_tokens or meta.positions.numel() < batch.num_tokens:
        raise ValueError("out_loc / positions hold fewer entries than the batch's new tokens")
    pt = _lib.PageTable(page_table.data_ptr(), page_table.shape[0], page_table.shape[1])
    m = meta.struct()
    return (ctypes.byref(b), ctypes.byref(pt), page_size, num_pool_rows,
            alloc_rows.data_ptr() if alloc_rows.numel() else None, alloc_rows.numel(), num_qo_heads, num_kv_heads,
            ctypes.byref(m)), (b, pt, m)


def build_attn_metadata(batch: BatchTensors, page_table: torch.Tensor, page_size: int, num_pool_rows: int,
                        alloc_rows: torch.Tensor, num_qo_heads: int, num_kv_heads: int, meta: MetadataBuffers,
                        stream=None) -> None:
    args, _keep = _metadata_args(batch, page_table, page_size, num_pool_rows, alloc_rows, num_qo_heads,
                                 num_kv_heads, meta)
    _check("build_attn_metadata", _lib.lib().build_attn_metadata(*args, _stream(stream)))


def _metadata_store_args(batch, page_table, pool, alloc_rows, num_qo_heads, meta, k_new, v_new):
    b = batch.struct()
    p = pool.struct()
    _need(page_table, "page_table", torch.int32, 2)
    _need(alloc_rows, "alloc_rows", torch.int32, 1)
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    if v_new.shape != k_new.shape or k_new.shape[1:] != pool.k.shape[1:] or k_new.shape[0] < batch.num_tokens:
        raise ValueError("k_new / v_new shapes do not match the batch and pool")
    if meta.out_loc.numel() < batch.num_tokens or meta.positions.numel() < batch.num_tokens:
        raise ValueError("out_loc / positions hold fewer entries than the batch's new tokens")
    pt = _lib.PageTable(page_table.data_ptr(), page_table.shape[0], page_table.shape[1])
    m = meta.struct()
    return (ctypes.byref(b), ctypes.byref(pt), ctypes.byref(p), alloc_rows.data_ptr() if alloc_rows.numel() else None,
            alloc_rows.numel(), num_qo_heads, ctypes.byref(m), k_new.data_ptr(), v_new.data_ptr()), (b, pt, p, m)


def build_attn_metadata_store(batch: BatchTensors, page_table: torch.Tensor, pool: KVPoolTensors,
                              alloc_rows: torch.Tensor, num_qo_heads: int, meta: MetadataBuffers, k_new: torch.Tensor,
                              v_new: torch.Tensor, stream=None) -> None:
    """build_attn_metadata followed by kv_store of k_new / v_new at the
    out_loc rows it writes, in one launch for batches of up to 1024 requests."""
    args, _keep = _metadata_store_args(batch, page_table, pool, alloc_rows, num_qo_heads, meta, k_new, v_new)
    _check("build_attn_metadata_store", _lib.lib().build_attn_metadata_store(*args, _stream(stream)))


def _attn_args(pool, page_table, batch, meta, q, o, sm_scale, workspace):
    p = pool.struct()
    b = batch.struct()
    _need(page_table, "page_table", torch.int32, 2)
    _need(q, "q", torch.bfloat16, 3)
    _need(o, "o", torch.bfloat16, 3)
    if q.shape != o.shape or q.shape[0] < batch.num_tokens or q.shape[2] != pool.k.shape[2]:
        raise ValueError("q / o shapes do not match the batch and pool")
    pt = _lib.PageTable(page_table.data_ptr(), page_table.shape[0], page_table.shape[1])
    m = meta.struct()
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", workspace.dtype, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return (ctypes.byref(p), ctypes.byref(pt), ctypes.byref(b), ctypes.byref(m), q.data_ptr(), o.data_ptr(),
            q.shape[1], float(sm_scale), ws_ptr, ws_bytes), (p, pt, b, m)


def _attn(fn_name, pool, page_table, batch, meta, q, o, sm_scale, workspace, stream):
    args, _keep = _attn_args(pool, page_table, batch, meta, q, o, sm_scale, workspace)
    _check(fn_name, getattr(_lib.lib(), fn_name)(*args, _stream(stream)))


def paged_decode_attn(pool: KVPoolTensors, page_table: torch.Tensor, batch: BatchTensors, meta: MetadataBuffers,
                      q: torch.Tensor, o: torch.Tensor, sm_scale: float, workspace: torch.Tensor,
                      stream=None) -> None:
    _attn("paged_decode_attn", pool, page_table, batch, meta, q, o, sm_scale, workspace, stream)


def paged_decode_attn_static(pool: KVPoolTensors, page_table: torch.Tensor, batch: BatchTensors,
                             meta: MetadataBuffers, q: torch.Tensor, o: torch.Tensor, sm_scale: float,
                             stream=None) -> None:
    """paged_decode_attn with the library's static device scratch as its
    workspace: allocates nothing (no device memory, no tensors).  Needs at most
    8 query heads per KV head; calls that overlap on one GPU race."""
    p = pool.struct()
    b = batch.struct()
    _need(page_table, "page_table", torch.int32, 2)
    _need(q, "q", torch.bfloat16, 3)
    _need(o, "o", torch.bfloat16, 3)
    if q.shape != o.shape or q.shape[0] < batch.num_tokens or q.shape[2] != pool.k.shape[2]:
        raise ValueError("q / o shapes do not match the batch and pool")
    pt = _lib.PageTable(page_table.data_ptr(), page_table.shape[0], page_table.shape[1])
    m = meta.struct()
    _check("paged_decode_attn_static",
           _lib.lib().paged_decode_attn_static(ctypes.byref(p), ctypes.byref(pt), ctypes.byref(b), ctypes.byref(m),
                                               q.data_ptr(), o.data_ptr(), q.shape[1], float(sm_scale),
                                               _stream(stream)))


def paged_extend_attn(pool: KVPoolTensors, page_table: torch.Tensor, batch: BatchTensors, meta: MetadataBuffers,
                      q: torch.Tensor, o: torch.Tensor, sm_scale: float, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    _attn("paged_extend_attn", pool, page_table, batch, meta, q, o, sm_scale, workspace, stream)


def rope_cos_sin_cache(cache: torch.Tensor, base: float, stream=None) -> None:
    """Fill cache (float32 [max_position, head_dim]) with the rotary table:
    cos(p theta_i) in the first half of row p, sin(p theta_i) in the second,
    theta_i = base^(-2i/head_dim)."""
    _need(cache, "cache", torch.float32, 2)
    if not cache.is_contiguous():
        raise ValueError("cache must be contiguous")
    _check("pkv_rope_cos_sin_cache", _lib.lib().pkv_rope_cos_sin_cache(cache.data_ptr(), cache.shape[0],
                                                                       cache.shape[1], float(base), _stream(stream)))


def kv_store_rope(pool: KVPoolTensors, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                  out_loc: torch.Tensor, positions: torch.Tensor, cos_sin_cache: torch.Tensor,
                  qk_norm: Optional[tuple] = None, status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Rotate q in place and k by positions (after the optional per-head RMS
    norm qk_norm = (q_weight, k_weight, eps)), then store k and v at out_loc."""
    p = pool.struct()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    _need(out_loc, "out_loc", torch.int32, 1)
    _need(positions, "positions", torch.int32, 1)
    _need(cos_sin_cache, "cos_sin_cache", torch.float32, 2)
    t = k_new.shape[0]
    if (v_new.shape != k_new.shape or k_new.shape[1:] != pool.k.shape[1:] or q.shape[0] < t
            or q.shape[2] != pool.k.shape[2] or out_loc.numel() < t or positions.numel() < t
            or cos_sin_cache.shape[1] != pool.k.shape[2]):
        raise ValueError("q / k_new / v_new / out_loc / positions / cache shapes do not match the pool")
    for name, x in (("q", q), ("k_new", k_new), ("v_new", v_new), ("cos_sin_cache", cos_sin_cache)):
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    norm = None
    if qk_norm is not None:
        qw, kw, eps = qk_norm
        _need(qw, "q_weight", torch.bfloat16, 1)
        _need(kw, "k_weight", torch.bfloat16, 1)
        norm = _lib.QKNorm(qw.data_ptr(), kw.data_ptr(), float(eps), 0)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    _check("kv_store_rope", _lib.lib().kv_store_rope(
        ctypes.byref(p), q.data_ptr(), q.shape[1], k_new.data_ptr(), v_new.data_ptr(), out_loc.data_ptr(),
        positions.data_ptr(), t, cos_sin_cache.data_ptr(), cos_sin_cache.shape[0],
        ctypes.byref(norm) if norm is not None else None, _ptr(status), _stream(stream)))


class BoundBatch:
    """A batch whose C struct is built once and shared by every call bound to
    it (bind_*): set_counts changes the request and token counts all of them
    see.  max_tokens (default: the batch's num_tokens) is the most new tokens
    a later set_counts may give; the bound calls' token buffers are checked
    against it when they are bound."""

    def __init__(self, batch: BatchTensors, max_tokens: Optional[int] = None):
        self.batch = batch
        self._struct = batch.struct()
        self.max_reqs = batch.table_idx.numel()
        self.max_tokens = batch.num_tokens if max_tokens is None else int(max_tokens)
        if self.max_tokens < batch.num_tokens:
            raise ValueError("max_tokens below the batch's num_tokens")

    def struct(self) -> _lib.Batch:
        return self._struct

    @property
    def num_tokens(self) -> int:
        """The token capacity bound calls' buffers must hold."""
        return self.max_tokens

    def set_counts(self, num_reqs: int, num_decode: int, num_tokens: int) -> None:
        """Requests [0, num_reqs) of the batch arrays, the first num_decode of
        them decode requests, with num_tokens new tokens in all."""
        if not (0 <= num_decode <= num_reqs <= self.max_reqs and 0 <= num_tokens <= self.max_tokens):
            raise ValueError(f"counts ({num_reqs}, {num_decode}, {num_tokens}) outside the bound batch "
                             f"({self.max_reqs} requests, {self.max_tokens} tokens)")
        s = self._struct
        s.num_reqs = num_reqs
        s.num_decode = num_decode
        s.num_tokens = num_tokens


class BoundCall:
    """One library call with its arguments checked and marshalled once.
    Calling it launches the call again on the bound stream (or the stream
    given): the buffers' contents may change between calls, their addresses
    may not (the bound call keeps the tensors alive), and the batch counts
    change through the BoundBatch it was bound to.  Per call it costs one
    ctypes call, against about 9 us of Python argument checks for the plain
    functions, so back-to-back eager steps of a small batch are bound by the
    GPU rather than by the host."""
    __slots__ = ("name", "_fn", "_args", "_stream", "_keep")

    def __init__(self, name, args, keep, stream):
        self.name = name
        self._fn = getattr(_lib.lib(), name)
        self._args = args
        self._keep = keep
        self._stream = _stream(stream)

    def __call__(self, stream=None) -> None:
        code = self._fn(*self._args, self._stream if stream is None else _stream(stream))
        if code != _lib.PKV_OK:
            raise PagedKVError(self.name, code)


def _bound_refs(*objs):
    return tuple(x for x in objs if x is not None)


def bind_kv_store(pool: KVPoolTensors, k_new: torch.Tensor, v_new: torch.Tensor, out_loc: torch.Tensor,
                  status: Optional[torch.Tensor] = None, stream=None) -> BoundCall:
    """kv_store bound once (see BoundCall); stores all k_new.shape[0] rows."""
    args, keep = _kv_store_args(pool, k_new, v_new, out_loc, status)
    return BoundCall("kv_store", args, keep + _bound_refs(pool, k_new, v_new, out_loc, status), stream)


def bind_build_attn_metadata(batch: BoundBatch, page_table: torch.Tensor, page_size: int, num_pool_rows: int,
                             alloc_rows: torch.Tensor, num_qo_heads: int, num_kv_heads: int, meta: MetadataBuffers,
                             stream=None) -> BoundCall:
    """build_attn_metadata bound once (see BoundCall)."""
    args, keep = _metadata_args(batch, page_table, page_size, num_pool_rows, alloc_rows, num_qo_heads,
                                num_kv_heads, meta)
    return BoundCall("build_attn_metadata", args, keep + _bound_refs(batch, page_table, alloc_rows, meta), stream)


def bind_build_attn_metadata_store(batch: BoundBatch, page_table: torch.Tensor, pool: KVPoolTensors,
                                   alloc_rows: torch.Tensor, num_qo_heads: int, meta: MetadataBuffers,
                                   k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> BoundCall:
    """build_attn_metadata_store bound once (see BoundCall)."""
    args, keep = _metadata_store_args(batch, page_table, pool, alloc_rows, num_qo_heads, meta, k_new, v_new)
    return BoundCall("build_attn_metadata_store", args,
                     keep + _bound_refs(batch, page_table, pool, alloc_rows, meta, k_new, v_new), stream)


def bind_paged_decode_attn(pool: KVPoolTensors, page_table: torch.Tensor, batch: BoundBatch, meta: MetadataBuffers,
                           q: torch.Tensor, o: torch.Tensor, sm_scale: float, workspace: torch.Tensor,
                           stream=None) -> BoundCall:
    """paged_decode_attn bound once (see BoundCall)."""
    args, keep = _attn_args(pool, page_table, batch, meta, q, o, sm_scale, workspace)
    return BoundCall("paged_decode_attn", args, keep + _bound_refs(pool, page_table, batch, meta, q, o, workspace),
                     stream)


def bind_paged_extend_attn(pool: KVPoolTensors, page_table: torch.Tensor, batch: BoundBatch, meta: MetadataBuffers,
                           q: torch.Tensor, o: torch.Tensor, sm_scale: float,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> BoundCall:
    """paged_extend_attn bound once (see BoundCall)."""
    args, keep = _attn_args(pool, page_table, batch, meta, q, o, sm_scale, workspace)
    return BoundCall("paged_extend_attn", args, keep + _bound_refs(pool, page_table, batch, meta, q, o, workspace),
                     stream)


class DecodeGraph:
    """The decode step (build_attn_metadata -> kv_store -> paged_decode_attn)
    captured as one HIP graph per batch size in `sizes` over fixed buffers
    sized for max_reqs requests; replay(n) pads to the smallest captured size
    >= n with dummy requests on `dummy_table_row` and launches that graph."""

    def __init__(self, pool: KVPoolTensors, page_table: torch.Tensor, batch: BatchTensors, alloc_rows: torch.Tensor,
                 q: torch.Tensor, o: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, meta: MetadataBuffers,
                 workspace: torch.Tensor, sm_scale: float, dummy_table_row: int, sizes, stream):
        if stream is None or _stream(stream) == 0:
            raise ValueError("graph capture needs a non-default stream")
        _need(page_table, "page_table", torch.int32, 2)
        _need(alloc_rows, "alloc_rows", torch.int32, 1)
        for name, x in (("q", q), ("o", o), ("k_new", k_new), ("v_new", v_new)):
            _need(x, name, torch.bfloat16, 3)
        max_reqs = batch.table_idx.numel()
        if (q.shape[0] < max_reqs or o.shape != q.shape or k_new.shape[0] < max_reqs or v_new.shape != k_new.shape
                or alloc_rows.numel() < max_reqs or batch.cached_len.numel() < max_reqs
                or batch.device_len.numel() < max_reqs):
            raise ValueError("graph buffers must hold max_reqs requests")
        _need(workspace, "workspace", workspace.dtype, 1)
        self._keep = (pool, page_table, batch, alloc_rows, q, o, k_new, v_new, meta, workspace)
        d = _lib.DecodeGraphDesc()
        d.pool = pool.struct()
        d.page_table = _lib.PageTable(page_table.data_ptr(), page_table.shape[0], page_table.shape[1])
        d.max_reqs = max_reqs
        d.dummy_table_row = dummy_table_row
        d.num_qo_heads = q.shape[1]
        d.sm_scale = float(sm_scale)
        d.table_idx, d.cached_len = batch.table_idx.data_ptr(), batch.cached_len.data_ptr()
        d.device_len, d.alloc_rows = batch.device_len.data_ptr(), alloc_rows.data_ptr()
        d.q, d.o, d.k_new, d.v_new = q.data_ptr(), o.data_ptr(), k_new.data_ptr(), v_new.data_ptr()
        d.meta = meta.struct()
        d.workspace = workspace.data_ptr()
        d.workspace_bytes = workspace.numel() * workspace.element_size()
        d.reserved = 0
        self.sizes = sorted(int(x) for x in sizes)
        arr = (ctypes.c_int32 * len(self.sizes))(*self.sizes)
        handle = ctypes.c_void_p()
        self._stream = stream
        _check("pkv_decode_graph_create",
               _lib.lib().pkv_decode_graph_create(ctypes.byref(d), arr, len(self.sizes), ctypes.byref(handle),
                                                  _stream(stream)))
        self._handle = handle

    def replay(self, num_reqs: int, stream=None) -> int:
        """Launch the graph for num_reqs real requests already written to the
        buffers' first slots (their new-page rows from alloc_rows[0] on);
        returns the padded batch size used."""
        bs = ctypes.c_int32(0)
        _check("pkv_decode_graph_replay",
               _lib.lib().pkv_decode_graph_replay(self._handle, num_reqs, ctypes.byref(bs),
                                                  _stream(stream or self._stream)))
        return bs.value

    def close(self) -> None:
        if getattr(self, "_handle", None) is not None and self._handle.value:
            _lib.lib().pkv_decode_graph_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


class PageFreeList:
    """A device-resident ring of free page-start rows (oldest first) that
    pkv_alloc_pages takes a batch's new pages from and pkv_free_pages appends
    to; its state (head, count) stays on the device."""

    def __init__(self, capacity: int, page_size: int, num_pool_rows: int, device="cuda"):
        self.rows = torch.zeros(capacity, dtype=torch.int32, device=device)
        self.state = torch.zeros(2, dtype=torch.int32, device=device)
        self.capacity, self.page_size, self.num_pool_rows = int(capacity), int(page_size), int(num_pool_rows)

    def struct(self) -> _lib.FreeList:
        return _lib.FreeList(self.rows.data_ptr(), self.state.data_ptr(), self.capacity, self.page_size,
                             self.num_pool_rows)

    def reset(self, free_rows: torch.Tensor, stream=None) -> None:
        """Start from free_rows (int32 page-start rows, oldest first)."""
        _need(free_rows, "free_rows", torch.int32, 1)
        n = free_rows.numel()
        if n > self.capacity:
            raise ValueError("more free rows than capacity")
        self.rows[:n].copy_(free_rows)
        f = self.struct()
        _check("pkv_free_list_reset", _lib.lib().pkv_free_list_reset(ctypes.byref(f), n, _stream(stream)))

    def alloc(self, batch: BatchTensors, alloc_rows: torch.Tensor, status: Optional[torch.Tensor] = None,
              stream=None) -> None:
        """The batch's new pages into alloc_rows (oldest free pages first, request by request)."""
        f, b = self.struct(), batch.struct()
        _need(alloc_rows, "alloc_rows", torch.int32, 1)
        if status is not None:
            _need(status, "status", torch.int32, 1)
        _check("pkv_alloc_pages", _lib.lib().pkv_alloc_pages(ctypes.byref(f), ctypes.byref(b), alloc_rows.data_ptr(),
                                                             alloc_rows.numel(), _ptr(status), _stream(stream)))

    def free(self, rows: torch.Tensor, status: Optional[torch.Tensor] = None, stream=None) -> None:
        f = self.struct()
        _need(rows, "rows", torch.int32, 1)
        if status is not None:
            _need(status, "status", torch.int32, 1)
        _check("pkv_free_pages", _lib.lib().pkv_free_pages(ctypes.byref(f), rows.data_ptr() if rows.numel() else None,
                                                           rows.numel(), _ptr(status), _stream(stream)))

    def snapshot(self):
        """The free rows, oldest first (host copy; synchronises)."""
        head, count = (int(x) for x in self.state.cpu())
        rows = self.rows.cpu().numpy()
        return [int(rows[(head + k) % self.capacity]) for k in range(count)]
