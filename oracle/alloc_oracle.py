"""Plain CPU oracle for the page allocator that feeds build_attn_metadata.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it and
shares no code with it.

What it follows: "mini-sglang learning notes" (doc-mini-sglang-learn), page-
table passage: the scheduler counts, page aligned, how many new pages each
request needs over [cached_len, device_len), takes them from free_slots in one
batch and writes them into the page table; free_slots is kept page aligned
(entries are page-start rows).  "mini-sglang architecture deep dive" §3.6: a
free list is a Python list, freed entries are appended.

Readings where the pages are silent: pages are taken from the front of the
free list, request by request in batch order, and freed pages are appended at
the back (first in, first out); a request whose lengths are not
0 <= cached_len <= device_len needs no page; when the list holds fewer pages
than the batch needs, nothing is taken (the caller evicts and retries).

Parity status: pinned by the tests (hand-worked batches, conservation and
order invariants, agreement with the pinned metadata oracle).  Not "parity
unpinned".
"""
from __future__ import annotations

from collections import deque
from typing import Iterable, List, Optional

import numpy as np


def new_pages(cached_len: int, device_len: int, page_size: int) -> int:
    """Pages to add so that [0, device_len) is covered when [0, cached_len) already is."""
    c, d, s = int(cached_len), int(device_len), int(page_size)
    if not (0 <= c <= d):
        return 0
    return -(-d // s) - (-(-c // s))


class FreeList:
    """Page-start rows not in use, oldest first."""

    def __init__(self, rows: Iterable[int], capacity: int):
        self.rows = deque(int(r) for r in rows)
        self.capacity = int(capacity)
        assert len(self.rows) <= self.capacity

    def allocate(self, cached_len, device_len, page_size: int) -> Optional[List[int]]:
        """The batch's new pages, request by request, or None (and no change)
        when the list holds too few."""
        need = sum(new_pages(c, d, page_size) for c, d in zip(cached_len, device_len))
        if need > len(self.rows):
            return None
        return [self.rows.popleft() for _ in range(need)]

    def free(self, rows: Iterable[int]) -> bool:
        rows = [int(r) for r in rows]
        if len(self.rows) + len(rows) > self.capacity:
            return False
        self.rows.extend(rows)
        return True

    def snapshot(self) -> np.ndarray:
        return np.array(self.rows, dtype=np.int64)
