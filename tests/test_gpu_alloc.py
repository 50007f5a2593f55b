"""GPU parity of the page allocator (pkv_free_list_reset / pkv_alloc_pages /
pkv_free_pages) against the oracle (oracle/alloc_oracle.py), through the C
ABI: every allocation's rows and the free list after every call are
bit-identical to the oracle's, across ring wrap-around, shortages, refused
frees, and into build_attn_metadata's page table."""
import numpy as np
import pytest
import torch

import paged_kv_attention_08_amd as pkv
import oracle.alloc_oracle as A
import oracle.pagedkv_oracle as O
from tests.gpu_harness import i32, log

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_batch(c, d):
    n = len(c)
    return pkv.BatchTensors(torch.zeros(n, dtype=torch.int32, device=DEV), i32(c, DEV), i32(d, DEV), n, 0)


@pytest.mark.parametrize("page_size", [1, 16, 64])
def test_alloc_free_sequence_matches_oracle(page_size):
    rng = np.random.default_rng(100 + page_size)
    npages, cap = 600, 300
    N = npages * page_size
    init = (rng.permutation(npages)[:250] * page_size).astype(np.int32)
    fl = pkv.PageFreeList(cap, page_size, N)
    fl.reset(i32(init, DEV))
    ref = A.FreeList(init.tolist(), cap)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    alloc = torch.full((4096,), -7, dtype=torch.int32, device=DEV)
    held = []
    log(f"allocator page_size {page_size}")
    for step in range(60):
        b = int(rng.integers(1, 24))
        c = rng.integers(0, 40 * page_size, size=b)
        d = c + rng.integers(0, 6 * page_size, size=b)
        if step % 7 == 3:
            c[0], d[0] = d[0] + 5, d[0]          # invalid lengths: no pages
        want = ref.allocate(c, d, page_size)
        fl.alloc(gpu_batch(c, d), alloc, status)
        torch.cuda.synchronize()
        if want is None:
            assert int(status.item()) & pkv.PKV_STATUS_OUT_OF_PAGES
            status.zero_()
        else:
            assert int(status.item()) == 0
            assert alloc[: len(want)].cpu().numpy().tolist() == want
            held += want
        assert fl.snapshot() == list(ref.snapshot())
        if step % 3 == 2 and held:
            k = int(rng.integers(1, len(held) + 1))
            pick = rng.permutation(len(held))[:k]
            ret = [held[i] for i in pick]
            held = [h for i, h in enumerate(held) if i not in set(pick.tolist())]
            assert ref.free(ret)
            fl.free(i32(ret, DEV), status)
            torch.cuda.synchronize()
            assert int(status.item()) == 0
            assert fl.snapshot() == list(ref.snapshot())


def test_shortage_maps_no_token_and_refused_frees():
    s, npages = 16, 64
    N = npages * s
    fl = pkv.PageFreeList(8, s, N)
    fl.reset(i32(np.arange(1, 6) * s, DEV))                  # 5 free pages
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    alloc = torch.full((16,), 3, dtype=torch.int32, device=DEV)
    c, d = np.array([0, 0]), np.array([48, 50])              # 3 + 4 = 7 pages > 5
    fl.alloc(gpu_batch(c, d), alloc, status)
    torch.cuda.synchronize()
    assert int(status.item()) == pkv.PKV_STATUS_OUT_OF_PAGES
    assert alloc[:7].cpu().tolist() == [-1] * 7 and alloc[7:].cpu().tolist() == [3] * 9
    assert fl.snapshot() == [16, 32, 48, 64, 80]
    # the metadata built on that allocation maps none of the new tokens
    pt = torch.zeros((3, 64), dtype=torch.int32, device=DEV)
    meta = pkv.MetadataBuffers.allocate(2, 98, 8, 8, DEV)
    meta.out_loc.fill_(1234)
    b = pkv.BatchTensors(i32([0, 1], DEV), i32(c, DEV), i32(d, DEV), 0, 98)
    pkv.build_attn_metadata(b, pt, s, N, alloc, 8, 8, meta)
    torch.cuda.synchronize()
    assert int(meta.status.item()) & pkv.PKV_STATUS_BAD_ALLOC
    assert (meta.out_loc[:98] == -1).all() and (meta.positions[:98] == -1).all()
    assert not pt.any()
    # refused frees leave the list as it was
    status.zero_()
    fl.free(i32([96, 112, 128, 144], DEV), status)           # 5 + 4 > capacity 8
    torch.cuda.synchronize()
    assert int(status.item()) == pkv.PKV_STATUS_FREE_OVERFLOW
    status.zero_()
    fl.free(i32([96, 100], DEV), status)                     # 100 is not page aligned
    torch.cuda.synchronize()
    assert int(status.item()) == pkv.PKV_STATUS_BAD_ALLOC
    assert fl.snapshot() == [16, 32, 48, 64, 80]


@pytest.mark.parametrize("page_size", [1, 16])
def test_alloc_feeds_metadata(page_size):
    """Cached pages, then the batch's new pages from the GPU allocator, then
    build_attn_metadata: page table, out_loc and positions equal the oracle's
    metadata on the oracle's allocation."""
    rng = np.random.default_rng(7 + page_size)
    s, R, W = page_size, 12, 1024
    npages = 4096 // s
    N = npages * s
    order = (rng.permutation(npages - 1) + 1) * s
    ref = A.FreeList(order.tolist(), npages)
    c = rng.integers(0, 300, size=R)
    d = c + rng.integers(1, 200, size=R)
    pt = np.zeros((R, W), dtype=np.int32)
    for r in range(R):                                       # cached pages, oldest free pages first
        for p in range(-(-int(c[r]) // s)):
            page = ref.allocate([0], [s], s)[0]
            pt[r, p * s:(p + 1) * s] = np.arange(page, page + s)
    fl = pkv.PageFreeList(npages, s, N)
    fl.reset(i32(ref.snapshot().astype(np.int32), DEV))
    want_alloc = ref.allocate(c, d, s)
    alloc = torch.zeros(4096, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    b = pkv.BatchTensors(i32(np.arange(R), DEV), i32(c, DEV), i32(d, DEV), 0, int((d - c).sum()))
    fl.alloc(b, alloc, status)
    pt_dev = i32(pt, DEV)
    meta = pkv.MetadataBuffers.allocate(R, b.num_tokens, 32, 8, DEV)
    pkv.build_attn_metadata(b, pt_dev, s, N, alloc[: len(want_alloc)], 32, 8, meta)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(meta.status.item()) == 0
    assert alloc[: len(want_alloc)].cpu().tolist() == want_alloc
    m = O.build_metadata(pt, np.arange(R), c, d, np.array(want_alloc, dtype=np.int64), s)
    T = b.num_tokens
    assert np.array_equal(pt_dev.cpu().numpy(), m["page_table"])
    assert np.array_equal(meta.out_loc[:T].cpu().numpy(), m["out_loc"])
    assert np.array_equal(meta.positions[:T].cpu().numpy(), m["positions"])
    assert fl.snapshot() == list(ref.snapshot())
