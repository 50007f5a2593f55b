"""Run the fp64 oracle over a whole synthetic workload.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).
The order follows the learning notes' store-then-attend description: the
page-table write and out_loc come first, then store_kv, then attention over
device_len keys per request.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np

from .pagedkv_oracle import KVPool, build_metadata, paged_attention, store_kv


def initial_pool(w) -> KVPool:
    """The pool before this batch: cached rows hold their K/V, the poison page
    reads NaN, everything else (the dummy page included) reads zero."""
    pool = KVPool(w.num_pool_rows, w.num_kv_heads, w.head_dim)
    pool.load(w.cached_rows.tolist(), w.k_cached, w.v_cached)
    pool.mark_poison(w.poison_rows)
    return pool


def reference_step(w, requests: Optional[Iterable[int]] = None,
                   tokens: Optional[Dict[int, Iterable[int]]] = None, attention: bool = True) -> dict:
    meta = build_metadata(w.page_table, w.table_idx, w.cached_len, w.device_len, w.alloc_rows, w.page_size)
    pool = store_kv(initial_pool(w), w.k_new, w.v_new, meta["out_loc"])
    out = {}
    if attention:
        out = paged_attention(pool, meta["page_table"], w.table_idx, w.cached_len, w.device_len, w.q,
                              w.num_kv_heads, w.sm_scale, requests=requests, tokens=tokens)
    return {"meta": meta, "pool": pool, "out": out}


def real_requests(w) -> np.ndarray:
    return np.nonzero(~w.is_padding)[0]
