"""Pins for the page-allocator oracle (oracle/alloc_oracle.py): hand-worked
batches, conservation and first-in-first-out order, and agreement with the
pinned metadata oracle (every new token lands in a page its request was
given)."""
from __future__ import annotations

import numpy as np

import oracle.alloc_oracle as A
import oracle.pagedkv_oracle as O


def pin_hand_worked():
    # page size 64; free pages at rows 64, 0, 128, 192, 256
    fl = A.FreeList([64, 0, 128, 192, 256], capacity=8)
    cached = [0, 64, 3, 64, 200]
    device = [65, 64, 64, 129, 4]   # 2 pages, 0, 0 (the cached page covers it), 2 (rows 128..191, 192), bad -> 0
    got = fl.allocate(cached, device, 64)
    assert got == [64, 0, 128, 192]
    assert list(fl.snapshot()) == [256]
    assert fl.allocate([0], [65], 64) is None          # needs 2, has 1: nothing taken
    assert list(fl.snapshot()) == [256]
    assert fl.free([7 * 64, 5 * 64])
    assert fl.allocate([0, 10], [1, 70], 64) == [256, 7 * 64]   # 1 + (2 - 1) pages, oldest first
    assert list(fl.snapshot()) == [5 * 64]
    fl2 = A.FreeList([0, 1, 2], capacity=3)
    assert not fl2.free([3])                           # over capacity: refused, unchanged
    assert list(fl2.snapshot()) == [0, 1, 2]
    # page size 1: one row per new token
    fl3 = A.FreeList(range(10, 20), capacity=10)
    assert fl3.allocate([5, 0, 7], [6, 3, 7], 1) == [10, 11, 12, 13]


def pin_conservation_and_order():
    rng = np.random.default_rng(5)
    s = 16
    pages = list(rng.permutation(1000)[:600] * s)
    fl = A.FreeList(pages, capacity=1000)
    taken = []
    for step in range(40):
        b = int(rng.integers(1, 12))
        c = rng.integers(0, 200, size=b)
        d = c + rng.integers(0, 80, size=b)
        got = fl.allocate(c, d, s)
        if got is None:
            continue
        assert len(got) == sum(-(-int(x) // s) - (-(-int(y) // s)) for x, y in zip(d, c))
        taken += got
        if step % 3 == 2 and taken:
            k = int(rng.integers(1, len(taken) + 1))
            ret, taken = taken[:k], taken[k:]
            assert fl.free(ret)
    # nothing lost, nothing duplicated
    assert sorted(taken + list(fl.snapshot())) == sorted(pages)
    # first in, first out: a freed page comes back only after the ones already free
    fl = A.FreeList([0, 16, 32], capacity=8)
    fl.free([48])
    assert fl.allocate([0, 0, 0, 0], [16, 16, 16, 16], 16) == [0, 16, 32, 48]


def pin_agrees_with_metadata():
    rng = np.random.default_rng(9)
    s, R, W, N = 16, 8, 512, 4096
    c = rng.integers(0, 200, size=R).astype(np.int64)
    d = c + rng.integers(1, 120, size=R)
    pt = np.zeros((R, W), dtype=np.int32)
    fl = A.FreeList(rng.permutation(N // s)[: N // s - 1] * s + s, capacity=N // s)
    # cached pages come from the list too, then the batch's new pages
    for r in range(R):
        ncached = -(-int(c[r]) // s)
        for p in range(ncached):
            page = fl.allocate([0], [s], s)[0]
            pt[r, p * s:(p + 1) * s] = np.arange(page, page + s)
    alloc = fl.allocate(c, d, s)
    meta = O.build_metadata(pt, np.arange(R), c, d, np.array(alloc, dtype=np.int64), s)
    off = 0
    for r in range(R):
        k = A.new_pages(c[r], d[r], s)
        mine = set(alloc[off:off + k])
        off += k
        for j in range(int(c[r]), int(d[r])):
            row = int(meta["page_table"][r, j])
            page = row - row % s
            if j >= -(-int(c[r]) // s) * s:                 # past the partial cached page
                assert page in mine
            else:
                assert page == int(pt[r, j - j % s])


ALL_PINS = [pin_hand_worked, pin_conservation_and_order, pin_agrees_with_metadata]
