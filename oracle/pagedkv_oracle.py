"""fp64 CPU oracle for the paged-KV attention step of one transformer layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it, and
it shares no code with the GPU library: no kernels, headers, helpers or table
generators.  It is deliberately plain and slow: explicit Python loops over
tokens and requests, an explicit gather through the page table, a naive
two-pass softmax in float64, and an explicit scatter.

What it follows (page titles and sections of the source pages):

* "mini-sglang architecture deep dive" (tinymind.me), §5.2 FlashAttention:
  attention is softmax(q·Kᵀ)·V; the tiled/online-softmax form only reorders
  that computation, so the oracle computes the untiled definition.
* same page, §5.3 PagedAttention: K/V live in a pool of physical blocks and
  each sequence reaches its tokens through its own table.
* same page, §6.1: per-token KV bytes = 2 (K and V) x layers x kv_heads x
  head_dim x dtype bytes (worked estimate 2x32x32x128x4096x2 B ~ 2 GB).
* "mini-sglang learning notes" (doc-mini-sglang-learn), passages on Req
  (cached_len, device_len, extend_len = device_len - cached_len), on the page
  table (one row per request, entry j = raw physical position of logical token
  j, width aligned up to 32, page-aligned allocation over
  [cached_len, device_len)), on store_kv (new K/V rows are scattered to the
  out_loc physical positions before attention runs) and on the dummy page.
* "SGLang source guide" (anrans.github.io), main line 3: ForwardBatch names
  seq_lens / extend_prefix_lens / extend_seq_lens / out_cache_loc for the same
  quantities.

Readings where the pages are silent (each is listed with its reason in the
design notes): consecutive query heads share a KV head (h // (Hq/Hkv)); the
causal alignment is bottom-right (new token t of a chunk sees keys
0 .. cached_len + t); the score scale is a plain multiplier with no soft-cap,
window or bias; new tokens first fill the request's partial last page.

Parity status: every function here is pinned by tests that do not re-type its
formula (library routines, closed forms, invariants, the pages' worked KV-size
figure).  No function is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional

import numpy as np


# ----------------------------------------------------------------------------
# bf16 handling
# ----------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# KV pool (one layer): physical row -> K row and V row, each [Hkv, d]
# ----------------------------------------------------------------------------

class KVPool:
    """The KV pool of one layer, keyed by physical row.

    mini-sglang allocates one big tensor per layer whose K and V buffers are
    (pages*page_size, kv_heads, head_dim) token-row arrays, the row number being
    the token's physical position (learning notes, KV-pool passage; deep dive
    §6.2).  Holding every row of a 150 GB pool in fp64 on the host is not
    possible, so this keeps only rows that were ever written; a row never
    written reads as zeros, and rows marked poison read as NaN.  Values are kept
    as bf16 bits and widened on gather.
    """

    def __init__(self, num_rows: int, num_kv_heads: int, head_dim: int):
        self.num_rows = int(num_rows)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self._index: Dict[int, int] = {}
        self._k: List[np.ndarray] = []
        self._v: List[np.ndarray] = []
        self._poison: set = set()

    def load(self, rows: Iterable[int], k_bits: np.ndarray, v_bits: np.ndarray) -> None:
        """Bulk initial contents: rows[n] holds k_bits[n], v_bits[n] ([Hkv, d] each).
        Rows are kept as read-only views of the given arrays."""
        k_bits = np.asarray(k_bits, dtype=np.uint16).reshape(-1, self.num_kv_heads, self.head_dim)
        v_bits = np.asarray(v_bits, dtype=np.uint16).reshape(-1, self.num_kv_heads, self.head_dim)
        for n, row in enumerate(rows):
            row = int(row)
            if not (0 <= row < self.num_rows):
                raise IndexError(f"pool row {row} outside [0, {self.num_rows})")
            self._poison.discard(row)
            if row in self._index:
                self._k[self._index[row]] = k_bits[n]
                self._v[self._index[row]] = v_bits[n]
            else:
                self._index[row] = len(self._k)
                self._k.append(k_bits[n])
                self._v.append(v_bits[n])

    def mark_poison(self, rows: Iterable[int]) -> None:
        self._poison.update(int(r) for r in rows)

    def write_row(self, row: int, k_row_bits: np.ndarray, v_row_bits: np.ndarray) -> None:
        if not (0 <= row < self.num_rows):
            raise IndexError(f"pool row {row} outside [0, {self.num_rows})")
        k = np.array(k_row_bits, dtype=np.uint16).reshape(self.num_kv_heads, self.head_dim)
        v = np.array(v_row_bits, dtype=np.uint16).reshape(self.num_kv_heads, self.head_dim)
        self._poison.discard(row)
        if row in self._index:
            self._k[self._index[row]] = k
            self._v[self._index[row]] = v
        else:
            self._index[row] = len(self._k)
            self._k.append(k)
            self._v.append(v)

    def row_bits(self, row: int):
        """(K bits, V bits) of one row, or None if the row was never written."""
        if row in self._index:
            n = self._index[row]
            return self._k[n], self._v[n]
        return None

    def gather(self, rows: List[int]):
        """Explicit gather of K[rows, :, :] and V[rows, :, :] in fp64 ([n, Hkv, d] each)."""
        n = len(rows)
        K = np.zeros((n, self.num_kv_heads, self.head_dim), dtype=np.float64)
        V = np.zeros((n, self.num_kv_heads, self.head_dim), dtype=np.float64)
        for a, row in enumerate(rows):
            if not (0 <= row < self.num_rows):
                raise IndexError(f"gather of pool row {row} outside [0, {self.num_rows})")
            if row in self._poison:
                K[a] = np.nan
                V[a] = np.nan
                continue
            got = self.row_bits(row)
            if got is not None:
                K[a] = widen_bf16(got[0])
                V[a] = widen_bf16(got[1])
        return K, V

    def copy(self) -> "KVPool":
        out = KVPool(self.num_rows, self.num_kv_heads, self.head_dim)
        out._index = dict(self._index)
        out._k = list(self._k)
        out._v = list(self._v)
        out._poison = set(self._poison)
        return out

    def written_rows(self) -> List[int]:
        return sorted(self._index)


# ----------------------------------------------------------------------------
# store_kv: scatter the batch's new K/V rows to out_loc
# ----------------------------------------------------------------------------

def store_kv(pool: KVPool, k_new_bits: np.ndarray, v_new_bits: np.ndarray, out_loc: np.ndarray) -> KVPool:
    """Each new token t's K row and V row go to physical row out_loc[t].

    Learning notes, store_kv passage: at every layer the attention backend first
    scatters the batch's freshly computed K/V to the pool at out_loc.  Tokens are
    taken in batch order, so if two tokens share a target (only padding requests
    do, on the dummy page) the later one wins here.
    """
    out = pool.copy()
    for t in range(len(out_loc)):
        out.write_row(int(out_loc[t]), k_new_bits[t], v_new_bits[t])
    return out


# ----------------------------------------------------------------------------
# build_attn_metadata: page-table write and per-batch indexing
# ----------------------------------------------------------------------------

def pages_needed(length: int, page_size: int) -> int:
    """Pages covering `length` tokens."""
    return -(-int(length) // int(page_size))


def build_metadata(page_table: np.ndarray, table_idx: np.ndarray, cached_len: np.ndarray,
                   device_len: np.ndarray, alloc_rows: np.ndarray, page_size: int) -> dict:
    """Write the new tokens' physical rows into the page table and derive the
    per-batch indexing.

    Learning notes, page-table passage: for each request the scheduler counts,
    page aligned, how many new pages [cached_len, device_len) needs, takes them
    from free_slots and writes the page table; entries are raw physical
    positions.  Reading of the partial-page case: a new token first fills the
    remaining slots of the request's last cached page (its row is that page's
    first row plus the slot), then the new pages in the order given.
    ``alloc_rows`` lists the first pool row of every new page, request by request.

    Returns the updated page table and, in batch order over new tokens:
    out_loc (physical row of each new token), positions (its logical index),
    qo_indptr / kv_indptr (running totals of extend_len and device_len, B+1
    entries starting at 0) and last_indices (index of each request's last new
    token).
    """
    s = int(page_size)
    pt = np.array(page_table, dtype=np.int64, copy=True)
    B = len(table_idx)
    out_loc: List[int] = []
    positions: List[int] = []
    qo_indptr = [0]
    kv_indptr = [0]
    cursor = 0
    for i in range(B):
        r = int(table_idx[i])
        c = int(cached_len[i])
        dl = int(device_len[i])
        first_new_page = pages_needed(c, s)
        for j in range(c, dl):
            logical_page = j // s
            slot = j % s
            if logical_page < first_new_page:
                row = int(pt[r, j - slot]) + slot
            else:
                row = int(alloc_rows[cursor + logical_page - first_new_page]) + slot
            pt[r, j] = row
            out_loc.append(row)
            positions.append(j)
        cursor += pages_needed(dl, s) - first_new_page
        qo_indptr.append(qo_indptr[-1] + (dl - c))
        kv_indptr.append(kv_indptr[-1] + dl)
    last_indices = [qo_indptr[i + 1] - 1 for i in range(B)]
    return {
        "page_table": pt.astype(np.int32),
        "out_loc": np.array(out_loc, dtype=np.int32),
        "positions": np.array(positions, dtype=np.int32),
        "qo_indptr": np.array(qo_indptr, dtype=np.int32),
        "kv_indptr": np.array(kv_indptr, dtype=np.int32),
        "last_indices": np.array(last_indices, dtype=np.int32),
        "alloc_used": cursor,
    }


# ----------------------------------------------------------------------------
# attention through the page table
# ----------------------------------------------------------------------------

def kv_head_of(h: int, group: int) -> int:
    """GQA: query head h reads KV head h // group (group = Hq / Hkv)."""
    return h // group


def keys_visible(cached_len: int, t: int) -> int:
    """New token t of a chunk sits at position cached_len + t and sees keys
    0 .. cached_len + t inclusive: the whole cached prefix plus the new rows up
    to itself (learning notes, Req and chunked-prefill passages)."""
    return cached_len + t + 1


def gather_rows(page_table: np.ndarray, table_row: int, n: int) -> List[int]:
    """Physical rows of logical tokens 0..n-1 of one request, entry by entry."""
    return [int(page_table[table_row, j]) for j in range(n)]


def scores(q_vec: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """s_j = scale * <q, k_j>."""
    return (K @ q_vec) * scale


def softmax(s: np.ndarray) -> np.ndarray:
    """Naive two-pass softmax: subtract the max, exponentiate, normalise."""
    m = np.max(s)
    e = np.exp(s - m)
    return e / np.sum(e)


def mix(p: np.ndarray, V: np.ndarray) -> np.ndarray:
    """o = sum_j p_j v_j."""
    return p @ V


def attend(q_vec: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q Kᵀ) V for one query vector (deep dive §5.2)."""
    return mix(softmax(scores(q_vec, K, scale)), V)


def attend_token(pool: KVPool, page_table: np.ndarray, table_row: int, n_keys: int, q_heads: np.ndarray,
                 num_kv_heads: int, scale: float) -> np.ndarray:
    """Output [Hq, d] of one new token that sees logical keys 0..n_keys-1."""
    Hq = q_heads.shape[0]
    group = Hq // num_kv_heads
    rows = gather_rows(page_table, table_row, n_keys)
    K_all, V_all = pool.gather(rows)
    out = np.empty((Hq, q_heads.shape[1]), dtype=np.float64)
    for h in range(Hq):
        g = kv_head_of(h, group)
        out[h] = attend(widen_bf16(q_heads[h]), K_all[:, g, :], V_all[:, g, :], scale)
    return out


def paged_attention(pool: KVPool, page_table: np.ndarray, table_idx: np.ndarray, cached_len: np.ndarray,
                    device_len: np.ndarray, q_bits: np.ndarray, num_kv_heads: int, scale: float,
                    requests: Optional[Iterable[int]] = None, tokens: Optional[Dict[int, Iterable[int]]] = None
                    ) -> Dict[int, np.ndarray]:
    """Attention of the batch's new tokens over their paged K/V (after store_kv).

    q rows are in batch order: request i's new tokens follow those of requests
    0..i-1.  Returns {global token index: [Hq, d] float64}.  ``requests``
    restricts the requests computed; ``tokens`` maps a request to the chunk
    offsets t to compute (default: all of them).
    """
    B = len(table_idx)
    req_set = set(range(B)) if requests is None else set(int(i) for i in requests)
    out: Dict[int, np.ndarray] = {}
    start = 0
    for i in range(B):
        c = int(cached_len[i])
        ext = int(device_len[i]) - c
        if i in req_set:
            offs = range(ext) if tokens is None or i not in tokens else tokens[i]
            for t in offs:
                out[start + t] = attend_token(pool, page_table, int(table_idx[i]), keys_visible(c, t),
                                              q_bits[start + t], num_kv_heads, scale)
        start += ext
    return out


# ----------------------------------------------------------------------------
# byte model
# ----------------------------------------------------------------------------

def kv_bytes(num_layers: int, num_kv_heads: int, head_dim: int, num_tokens: int, dtype_bytes: int) -> int:
    """KV-cache bytes of `num_tokens` tokens: K and V for every layer, KV head and
    head dimension (deep dive §6.1 estimate; learning notes, pool-sizing passage)."""
    return 2 * num_layers * num_kv_heads * head_dim * num_tokens * dtype_bytes


def decode_step_bytes(device_lens: Iterable[int], num_qo_heads: int, num_kv_heads: int, head_dim: int,
                      page_size: int, dtype_bytes: int = 2) -> int:
    """Bytes a decode pass over these requests must move at least once: every
    visible K and V row of one layer, one page-table entry per page (per token at
    page_size 1), the query and the output."""
    total = 0
    for dl in device_lens:
        dl = int(dl)
        entries = dl if page_size == 1 else pages_needed(dl, page_size)
        total += kv_bytes(1, num_kv_heads, head_dim, dl, dtype_bytes) + 4 * entries \
            + 2 * num_qo_heads * head_dim * dtype_bytes
    return total


def store_bytes(num_tokens: int, num_kv_heads: int, head_dim: int, dtype_bytes: int = 2) -> int:
    """kv_store moves each new K and V row in and out once and reads out_loc."""
    return num_tokens * (2 * kv_bytes(1, num_kv_heads, head_dim, 1, dtype_bytes) + 4)


def extend_flops(cached_len: Iterable[int], device_len: Iterable[int], num_qo_heads: int, head_dim: int) -> int:
    """Useful flops of extend attention: 2*d for q·k and 2*d for p·v per
    visible (query head, key) pair; exponentials not counted."""
    pairs = 0
    for c, dl in zip(cached_len, device_len):
        c, dl = int(c), int(dl)
        for t in range(dl - c):
            pairs += keys_visible(c, t)
    return 4 * num_qo_heads * head_dim * pairs
