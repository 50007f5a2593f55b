"""Algorithmic work of the paged-KV step (what the method must move or compute
at least once), used to turn measured times into GB/s, TFLOP/s and roofline
fractions.  Padding requests, split-K workspace traffic, masked-tile waste and
the softmax exponentials are not counted.

Per-token KV bytes follow "mini-sglang architecture deep dive" §6.1 (2 x
layers x KV heads x head_dim x dtype bytes; one layer here).
"""
from __future__ import annotations

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
BF16_DENSE_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz


def decode_bytes(device_len, num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                 dtype_bytes: int = 2) -> int:
    """K and V rows of every visible key, one int32 page-table entry per page
    (per key at page size 1), the query row and the output row."""
    dl = np.asarray(device_len, dtype=np.int64)
    entries = dl if page_size == 1 else -(-dl // page_size)
    kv = 2 * num_kv_heads * head_dim * dtype_bytes * dl
    qo = 2 * num_qo_heads * head_dim * dtype_bytes
    return int((kv + 4 * entries + qo).sum())


def store_bytes(num_tokens: int, num_kv_heads: int, head_dim: int, dtype_bytes: int = 2) -> int:
    """Read k_new and v_new, write both pool rows, read out_loc."""
    return int(num_tokens) * (4 * num_kv_heads * head_dim * dtype_bytes + 4)


def metadata_bytes(num_reqs: int, num_tokens: int) -> int:
    """Read table_idx / cached_len / device_len and one alloc entry per new
    token (upper bound at page size 1); write page-table entry, out_loc and
    position per token, two running totals and last_indices per request."""
    return int(num_reqs) * (3 * 4 + 3 * 4) + int(num_tokens) * (4 + 3 * 4) + 8


def extend_flops(cached_len, device_len, num_qo_heads: int, head_dim: int) -> int:
    """4 * d flops (q.k and p.v) per visible (query head, key) pair; new token t
    of a chunk sees cached_len + t + 1 keys."""
    c = np.asarray(cached_len, dtype=np.int64)
    n = np.asarray(device_len, dtype=np.int64) - c
    pairs = (n * c + n * (n + 1) // 2).sum()
    return int(4 * num_qo_heads * head_dim * pairs)


def rope_store_bytes(num_tokens: int, num_qo_heads: int, num_kv_heads: int, head_dim: int,
                     qk_norm: bool = True) -> int:
    """kv_store_rope: q read and written, k and v read, two pool rows written,
    out_loc and positions read, one float table row (head_dim floats) per
    token, the two norm weight rows once."""
    t = int(num_tokens)
    q = 2 * t * num_qo_heads * head_dim * 2
    kv = 2 * t * num_kv_heads * head_dim * 2
    return q + 2 * kv + 8 * t + t * head_dim * 4 + (2 * head_dim * 2 if qk_norm else 0)


def extend_unique_bytes(page_table, table_idx, cached_len, device_len, num_qo_heads: int, num_kv_heads: int,
                        head_dim: int, page_size: int, dtype_bytes: int = 2) -> int:
    """Bytes an extend pass must move at least once: every distinct K and V
    row its requests see (a radix-shared prefix once; the batch's new rows
    included), one page-table entry per visible key (per page at page size
    > 1), and each new token's query and output rows.  page_table is the state
    before the batch (cached entries only): new rows are distinct by
    construction and counted by number."""
    rows = set()
    entries = 0
    new = 0
    for r, c, dl in zip(table_idx, cached_len, device_len):
        c, dl = int(c), int(dl)
        rows.update(np.asarray(page_table[int(r), :c], dtype=np.int64).tolist())
        new += dl - c
        entries += dl if page_size == 1 else -(-dl // page_size)
    kv = (len(rows) + new) * 2 * num_kv_heads * head_dim * dtype_bytes
    return int(kv + 4 * entries + new * 2 * num_qo_heads * head_dim * dtype_bytes)
