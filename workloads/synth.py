"""Seeded synthetic inputs for the paged-KV attention step.

This module only *draws* inputs: request lengths, which physical pool rows hold
each request's cached tokens, which pages the scheduler hands out for new
tokens, and the N(0,1) q / k / v values rounded to bf16.  It computes none of
the attention step itself: no page-table write for new tokens, no out_loc, no
prefix sums, no softmax.  Both the fp64 oracle and the GPU path consume what
it returns.

Vocabulary follows the mini-sglang Req/Batch model (doc-mini-sglang-learn,
"Req" and "page table" passages; mini-sglang architecture deep dive §3.6 and
§6.2):

* ``cached_len``   tokens already in the KV pool (prefix hit + earlier chunks)
* ``device_len``   tokens the request covers after this forward
* ``extend_len``   ``device_len - cached_len`` new tokens in this batch
* ``page_table``   int32 ``[R, W]``; row ``table_idx[i]`` holds, at column j,
  the *raw physical pool row* of logical token j; ``W`` is a multiple of 32
* page ``p`` owns pool rows ``[p*s, (p+1)*s)`` for page size ``s``
* page 0 is the dummy page: padded requests read and write only there
* the last page is never handed out; its rows are NaN ("poison") and every
  page-table entry at or beyond a request's ``cached_len`` points into it, so
  a kernel that reads past ``device_len`` produces NaN.

The draw order for one workload is fixed: lengths, physical pages, q, k_new,
v_new, cached K, cached V; each stage has its own child ``SeedSequence`` so a
stage's values do not depend on how many numbers an earlier stage drew.
Large normal fills are split into fixed-size chunks, each with its own child
seed, so the result is the same for any thread count.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
_CHUNK_ELEMS = 1 << 22  # elements per independently seeded normal chunk


def float32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs here are finite N(0,1) draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_float32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32 (used only for display and tests)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_chunk(args):
    seed_seq, out_slice = args
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    tmp = rng.standard_normal(out_slice.size, dtype=np.float32)
    out_slice[...] = float32_to_bf16_bits(tmp).reshape(out_slice.shape)


def normal_bf16(seed_seq: np.random.SeedSequence, shape: Sequence[int], threads: int = 8) -> np.ndarray:
    """N(0,1) values rounded to bf16, as uint16 bits, filled chunk by chunk."""
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    n = out.size
    nchunks = max(1, math.ceil(n / _CHUNK_ELEMS))
    seeds = seed_seq.spawn(nchunks)
    jobs = [(seeds[c], out[c * _CHUNK_ELEMS:min(n, (c + 1) * _CHUNK_ELEMS)]) for c in range(nchunks)]
    if nchunks == 1 or threads <= 1:
        for j in jobs:
            _fill_chunk(j)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(_fill_chunk, jobs))
    return out.reshape(shape)


def align_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


@dataclass
class RequestSpec:
    """Lengths of one request in the batch (host-side scheduler state)."""
    cached_len: int
    device_len: int
    padding: bool = False          # a dummy request that only fills the batch
    shared_prefix: int = 0         # leading cached tokens that live in the shared prefix rows


@dataclass
class Workload:
    """One batch of one layer's attention step, ready for either side."""
    name: str
    seed: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pool_rows: int
    sm_scale: float
    num_decode: int                 # first num_decode requests have extend_len == 1
    table_idx: np.ndarray           # int32 [B]
    cached_len: np.ndarray          # int32 [B]
    device_len: np.ndarray          # int32 [B]
    is_padding: np.ndarray          # bool [B]
    page_table: np.ndarray          # int32 [R, W], state *before* this batch's write
    alloc_rows: np.ndarray          # int32 [sum new pages]: first pool row of each new page
    q: np.ndarray                   # bf16 bits [T, Hq, d], rows in batch order
    k_new: np.ndarray               # bf16 bits [T, Hkv, d]
    v_new: np.ndarray               # bf16 bits [T, Hkv, d]
    cached_rows: np.ndarray         # int64 [M] distinct pool rows holding cached tokens
    k_cached: np.ndarray            # bf16 bits [M, Hkv, d]
    v_cached: np.ndarray            # bf16 bits [M, Hkv, d]
    dummy_table_row: int
    notes: dict = field(default_factory=dict)

    @property
    def num_reqs(self) -> int:
        return int(self.table_idx.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def width(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def dummy_rows(self) -> range:
        return range(0, self.page_size)

    @property
    def poison_rows(self) -> range:
        return range(self.num_pool_rows - self.page_size, self.num_pool_rows)

    @property
    def extend_len(self) -> np.ndarray:
        return (self.device_len - self.cached_len).astype(np.int64)

    def summary(self) -> str:
        return (f"{self.name}: B={self.num_reqs} (decode {self.num_decode}, padding {int(self.is_padding.sum())}) "
                f"T={self.num_tokens} Hq={self.num_qo_heads} Hkv={self.num_kv_heads} d={self.head_dim} "
                f"s={self.page_size} N={self.num_pool_rows} W={self.width}")


def _draw_pages(rng: np.random.Generator, num_pages: int, count: int, order: str = "random") -> np.ndarray:
    """`count` distinct free pages, never page 0 (dummy) or the last page (poison).

    order "random": a seeded random order of all free pages (rows scattered over
    the whole pool, as after long churn).  order "sequential": pages 1, 2, ... in
    allocation order, as a fresh pool's free list hands them out."""
    free = num_pages - 2
    if count > free:
        raise ValueError(f"pool too small: need {count} pages, have {free} free")
    if order == "sequential":
        return np.arange(1, count + 1, dtype=np.int64)
    if order != "random":
        raise ValueError(f"unknown page order {order!r}")
    if free <= (1 << 24):
        return rng.permutation(free)[:count].astype(np.int64) + 1
    return rng.choice(free, size=count, replace=False, shuffle=True).astype(np.int64) + 1


def build_workload(name: str, seed: int, reqs: List[RequestSpec], *, num_qo_heads: int, num_kv_heads: int,
                   head_dim: int, page_size: int, num_pool_rows: int, num_decode: int,
                   width: Optional[int] = None, spare_table_rows: int = 1, threads: int = 8,
                   page_order: str = "random") -> Workload:
    """Lay out a batch in a paged pool and draw its values.

    Physical layout: a shared prefix (if any request has ``shared_prefix``) gets
    its pages first; then each non-padding request gets its private cached pages
    followed by its newly allocated pages, all drawn from one seeded random
    order of the free pages.  Padding requests point at the dummy page and a
    dedicated all-zero table row.
    """
    s = page_size
    if num_pool_rows % s:
        raise ValueError("num_pool_rows must be a multiple of page_size")
    num_pages = num_pool_rows // s
    root = np.random.SeedSequence(seed)
    ss_len_unused, ss_pages, ss_q, ss_k, ss_v, ss_kc, ss_vc, ss_tab = root.spawn(8)

    B = len(reqs)
    real = [i for i, r in enumerate(reqs) if not r.padding]
    shared = max([r.shared_prefix for r in reqs] + [0])
    if shared % s:
        raise ValueError("a shared prefix must be page aligned")
    for r in reqs:
        if r.shared_prefix not in (0, shared):
            raise ValueError("one shared prefix per batch")
        if r.shared_prefix > r.cached_len or r.cached_len > r.device_len:
            raise ValueError("lengths must satisfy shared_prefix <= cached_len <= device_len")
        if r.padding and (r.cached_len, r.device_len) != (0, 1):
            raise ValueError("padding requests have cached_len 0 and device_len 1")
    max_dev = max([r.device_len for r in reqs] + [1])
    W = width if width is not None else align_up(max_dev, 32)
    if W % 32 or W < max_dev:
        raise ValueError("page-table width must be a multiple of 32 covering every device_len")

    # --- physical pages -------------------------------------------------------
    shared_pages = shared // s
    priv_cached = {i: math.ceil(reqs[i].cached_len / s) - reqs[i].shared_prefix // s for i in real}
    new_pages = {i: math.ceil(reqs[i].device_len / s) - math.ceil(reqs[i].cached_len / s) for i in real}
    total = shared_pages + sum(priv_cached.values()) + sum(new_pages.values())
    rng_pages = np.random.Generator(np.random.PCG64(ss_pages))
    order = _draw_pages(rng_pages, num_pages, total, page_order)
    cur = 0
    shared_list = order[cur:cur + shared_pages]; cur += shared_pages
    req_cached_pages, req_new_pages = {}, {}
    for i in real:
        req_cached_pages[i] = np.concatenate([shared_list if reqs[i].shared_prefix else shared_list[:0],
                                              order[cur:cur + priv_cached[i]]]); cur += priv_cached[i]
        req_new_pages[i] = order[cur:cur + new_pages[i]]; cur += new_pages[i]

    # --- page table (state before this batch) ----------------------------------
    R = len(real) + spare_table_rows + 1
    dummy_row = R - 1
    rng_tab = np.random.Generator(np.random.PCG64(ss_tab))
    rows_for_real = rng_tab.permutation(R - 1)[:len(real)]
    poison_base = (num_pages - 1) * s
    pt = np.empty((R, W), dtype=np.int32)
    pt[:] = (poison_base + (np.arange(W) % s)).astype(np.int32)[None, :]
    pt[dummy_row, :] = 0
    table_idx = np.full(B, dummy_row, dtype=np.int32)
    cached_rows_list = []
    seen_shared = False
    for k, i in enumerate(real):
        r = int(rows_for_real[k])
        table_idx[i] = r
        cl = reqs[i].cached_len
        if cl:
            j = np.arange(cl)
            pages = req_cached_pages[i]
            phys = pages[j // s] * s + (j % s)
            pt[r, :cl] = phys.astype(np.int32)
            if reqs[i].shared_prefix:
                if not seen_shared:
                    cached_rows_list.append(phys[:shared])
                    seen_shared = True
                cached_rows_list.append(phys[shared:])
            else:
                cached_rows_list.append(phys)
    cached_rows = (np.concatenate(cached_rows_list) if cached_rows_list else np.zeros(0, np.int64)).astype(np.int64)
    assert np.unique(cached_rows).size == cached_rows.size

    alloc = []
    for i in range(B):
        if reqs[i].padding:
            alloc.append(np.zeros(1, np.int64))           # the dummy page
        else:
            alloc.append(req_new_pages[i] * s)
    alloc_rows = (np.concatenate(alloc) if alloc else np.zeros(0, np.int64)).astype(np.int32)

    cached_len = np.array([r.cached_len for r in reqs], dtype=np.int32)
    device_len = np.array([r.device_len for r in reqs], dtype=np.int32)
    T = int((device_len.astype(np.int64) - cached_len).sum())
    Hq, Hkv, d = num_qo_heads, num_kv_heads, head_dim
    q = normal_bf16(ss_q, (T, Hq, d), threads)
    k_new = normal_bf16(ss_k, (T, Hkv, d), threads)
    v_new = normal_bf16(ss_v, (T, Hkv, d), threads)
    k_cached = normal_bf16(ss_kc, (cached_rows.size, Hkv, d), threads)
    v_cached = normal_bf16(ss_vc, (cached_rows.size, Hkv, d), threads)
    return Workload(name=name, seed=seed, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=d, page_size=s,
                    num_pool_rows=num_pool_rows, sm_scale=1.0 / math.sqrt(d), num_decode=num_decode,
                    table_idx=table_idx, cached_len=cached_len, device_len=device_len,
                    is_padding=np.array([r.padding for r in reqs], dtype=bool), page_table=pt,
                    alloc_rows=alloc_rows, q=q, k_new=k_new, v_new=v_new, cached_rows=cached_rows,
                    k_cached=k_cached, v_cached=v_cached, dummy_table_row=dummy_row)
