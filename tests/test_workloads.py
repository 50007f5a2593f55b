"""CPU tests of the seeded input generators (structure only; no attention arithmetic)."""
import numpy as np
import pytest
import torch

from workloads import configs, float32_to_bf16_bits, normal_bf16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.0078125, 3.0e-39, 65504.0], dtype=np.float32)])
    ours = float32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_normal_fill_is_thread_count_independent():
    a = normal_bf16(np.random.SeedSequence(5), (3, 1 << 21), threads=1)
    b = normal_bf16(np.random.SeedSequence(5), (3, 1 << 21), threads=8)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_small_workload_structure(cfg):
    w = configs.small(cfg)
    s = w.page_size
    assert w.width % 32 == 0 and w.width >= w.device_len.max()
    assert w.num_pool_rows % s == 0
    # cached entries are raw rows; within a page consecutive slots are consecutive rows
    for i in range(w.num_reqs):
        r, c = w.table_idx[i], int(w.cached_len[i])
        if w.is_padding[i]:
            assert r == w.dummy_table_row and c == 0 and w.device_len[i] == 1
            continue
        rows = w.page_table[r, :c].astype(np.int64)
        j = np.arange(c)
        assert np.all(rows - rows[j - j % s] == j % s)
        assert np.all(rows[j - j % s] % s == 0)
        assert not np.any(np.isin(rows, list(w.dummy_rows) + list(w.poison_rows)))
        tail = w.page_table[r, c:]
        assert np.all(np.isin(tail, list(w.poison_rows)))
    assert np.all(w.page_table[w.dummy_table_row] == 0)
    assert np.all(w.alloc_rows % s == 0)
    real_alloc = w.alloc_rows[w.alloc_rows != 0]
    assert np.unique(real_alloc).size == real_alloc.size
    assert not np.any(np.isin(real_alloc, w.cached_rows))
    # decode requests come first and have one new token
    assert np.all(w.device_len[:w.num_decode] - w.cached_len[:w.num_decode] == 1)
    assert w.q.shape == (w.num_tokens, w.num_qo_heads, w.head_dim)
    assert w.k_new.shape == (w.num_tokens, w.num_kv_heads, w.head_dim)


def test_shared_prefix_rows_are_shared():
    w = configs.small(3)
    rows = [w.page_table[w.table_idx[i], :96] for i in range(w.num_reqs)]
    for r in rows[1:]:
        assert np.array_equal(r, rows[0])


@pytest.mark.parametrize("page_size", [1, 64])
def test_sequential_page_order(page_size):
    """Allocation-order pages: the same batch as the random order, with the pages
    handed out 1, 2, 3, ... (prefix first, then each request's cached and new pages)."""
    if page_size == 1:
        kw = dict(nreq=3, prefix=96, tail_hi=70, chunk=83, num_pool_rows=1 << 13)
        seq = configs.extend_radix(page_order="sequential", **kw)
        rnd = configs.extend_radix(**kw)
    else:
        kw = dict(ndec=6, dec_lo=1, dec_hi=300, next_=3, pre_hi=200, new_tokens=150, num_pool_rows=64 * 64)
        seq = configs.mixed_page64(page_order="sequential", **kw)
        rnd = configs.mixed_page64(**kw)
    assert np.array_equal(seq.cached_len, rnd.cached_len) and np.array_equal(seq.device_len, rnd.device_len)
    assert np.array_equal(seq.q, rnd.q)
    s = page_size
    pages = []
    for i in range(seq.num_reqs):
        if seq.is_padding[i]:
            continue
        r, c = seq.table_idx[i], int(seq.cached_len[i])
        pages.append(seq.page_table[r, :c:s].astype(np.int64) // s)
    allp = np.concatenate(pages + [seq.alloc_rows[seq.alloc_rows != 0].astype(np.int64) // s])
    uniq = np.unique(allp)
    assert np.array_equal(uniq, np.arange(1, uniq.size + 1))   # pages 1..n, none skipped
    with pytest.raises(ValueError):
        configs.extend_radix(page_order="sorted", **dict(nreq=2, prefix=32, tail_hi=8, chunk=8,
                                                          num_pool_rows=1 << 10))
