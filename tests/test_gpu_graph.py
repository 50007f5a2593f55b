"""GPU tests of the graph-replayed decode step (pkv_decode_graph_*), through
the C ABI: every replay's real outputs are bit-identical to the same padded
batch run eagerly through the three calls, and within the attention bar of
the fp64 oracle; replays of several padded sizes are interleaved with eager
work and repeated (graph nodes must give the same result on every replay).
Around every replay the whole pool is compared with a copy taken before it:
only the real requests' new rows and the dummy page may change, also at page
size 16, where the real requests need fewer new pages than there are requests
and earlier, larger batches have left other rows in alloc_rows past them."""
import numpy as np
import pytest
import torch

import paged_kv_attention_08_amd as pkv
from tests import parity_checks as P
from tests.gpu_harness import DeviceStep, bf16_tensor, i32, log
from workloads import RequestSpec, build_workload

pytestmark = pytest.mark.gpu
SIZES = [1, 2, 4, 8, 16]


def device_step(w):
    ds = DeviceStep(w)
    # one new page at most per decode request: room for max_reqs alloc entries
    ds.alloc_rows = torch.zeros(w.num_reqs, dtype=torch.int32, device=ds.device)
    return ds


def decode_workload(seed, page_size, nreq=16, num_pool_rows=1 << 14):
    rng = np.random.default_rng(seed)
    reqs = [RequestSpec(int(L), int(L) + 1) for L in rng.integers(40, 400, size=nreq)]
    return build_workload("graph_decode", seed, reqs, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          page_size=page_size, num_pool_rows=num_pool_rows, num_decode=nreq)


def new_pages(w, n):
    s = w.page_size
    dl, cl = w.device_len[:n].astype(np.int64), w.cached_len[:n].astype(np.int64)
    return int(((dl + s - 1) // s - (cl + s - 1) // s).sum())


def write_real(ds, w, n):
    """The first n requests of w into slots [0, n) of the fixed buffers."""
    dev = ds.device
    ds.batch.table_idx[:n].copy_(i32(w.table_idx[:n], dev))
    ds.batch.cached_len[:n].copy_(i32(w.cached_len[:n], dev))
    ds.batch.device_len[:n].copy_(i32(w.device_len[:n], dev))
    na = new_pages(w, n)
    ds.alloc_rows[:na].copy_(i32(w.alloc_rows[:na], dev))
    ds.q[:n].copy_(bf16_tensor(w.q[:n], dev))
    ds.k_new[:n].copy_(bf16_tensor(w.k_new[:n], dev))
    ds.v_new[:n].copy_(bf16_tensor(w.v_new[:n], dev))
    return na


def eager_padded(ds, w, n, bs, stream):
    """The same padded batch of bs requests through the three calls."""
    dev = ds.device
    na = write_real(ds, w, n)
    pad = bs - n
    torch.cuda.synchronize()
    if pad:
        ds.batch.table_idx[n:bs].fill_(int(w.dummy_table_row))
        ds.batch.cached_len[n:bs].fill_(0)
        ds.batch.device_len[n:bs].fill_(1)
        ds.alloc_rows[na:na + pad].fill_(0)
    torch.cuda.synchronize()
    b = pkv.BatchTensors(ds.batch.table_idx[:bs], ds.batch.cached_len[:bs], ds.batch.device_len[:bs], bs, bs)
    with torch.cuda.stream(stream):
        pkv.build_attn_metadata(b, ds.page_table, w.page_size, w.num_pool_rows, ds.alloc_rows[:bs], w.num_qo_heads,
                                w.num_kv_heads, ds.meta, stream=stream)
        pkv.kv_store(ds.pool, ds.k_new[:bs], ds.v_new[:bs], ds.meta.out_loc[:bs], ds.meta.status, stream=stream)
        pkv.paged_decode_attn(ds.pool, ds.page_table, b, ds.meta, ds.q[:bs], ds.o[:bs], w.sm_scale, ds.workspace,
                              stream=stream)
    stream.synchronize()
    return ds.o[:n].clone()


# (page size, captured sizes, requests, replayed batch sizes in order); the
# 520-request graph maps its tokens in build_attn_metadata's second kernel
CASES = {"page1": (1, SIZES, 16, (16, 5, 1, 8, 3, 16, 5)),
         "page16": (16, SIZES, 16, (16, 5, 1, 8, 3, 16, 5)),
         "page16_520": (16, [8, 520], 520, (520, 300, 7, 520, 301))}


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replay_matches_eager_and_oracle(case):
    page_size, sizes, nreq, order = CASES[case]
    w = decode_workload(41 + page_size + nreq, page_size, nreq, 1 << 14 if nreq <= 16 else 1 << 17)
    log(f"decode graph {case}: {w.summary()}")
    ds = device_step(w)
    stream = torch.cuda.Stream()
    ref = P.oracle_for(w)
    graph = pkv.DecodeGraph(ds.pool, ds.page_table, ds.batch, ds.alloc_rows, ds.q, ds.o, ds.k_new, ds.v_new,
                            ds.meta, ds.workspace, w.sm_scale, int(w.dummy_table_row), sizes, stream)
    try:
        for n in order:
            bs = next(s for s in sizes if s >= n)
            want = eager_padded(ds, w, n, bs, stream)
            ds.o.fill_(float("nan"))
            torch.cuda.synchronize()
            allowed = np.zeros(w.num_pool_rows, dtype=bool)
            allowed[ref["meta"]["out_loc"][:n]] = True
            allowed[w.dummy_rows.start:w.dummy_rows.stop] = True
            for rep in range(3):
                write_real(ds, w, n)
                torch.cuda.synchronize()
                before = ds.snapshot_pool()
                got_bs = graph.replay(n, stream=stream)
                stream.synchronize()
                assert got_bs == bs
                P.check_pool_unchanged_elsewhere(ds, before, allowed)
                k, v = ds.pool_rows_bits(ref["meta"]["out_loc"][:n])
                assert np.array_equal(k, w.k_new[:n]) and np.array_equal(v, w.v_new[:n]), "stored rows"
                del before
                got = ds.o[:n].clone()
                assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"n={n} replay {rep} != eager"
                # eager work on the default stream between replays
                torch.cuda.synchronize()
                _ = (ds.q.float().sum() + 1).item()
            assert ds.status() == 0
            stats = P.check_attention(ds, {i: ref["out"][i] for i in range(n)}, w, f"graph n={n}")
            log(f"n={n} bs={bs} max-abs {stats['max_abs']:.2e}")
    finally:
        graph.close()
        ds.free()


def test_graph_rejects_batches_beyond_the_largest_size():
    w = decode_workload(77, 1)
    ds = device_step(w)
    stream = torch.cuda.Stream()
    graph = pkv.DecodeGraph(ds.pool, ds.page_table, ds.batch, ds.alloc_rows, ds.q, ds.o, ds.k_new, ds.v_new,
                            ds.meta, ds.workspace, w.sm_scale, int(w.dummy_table_row), [1, 2, 4], stream)
    try:
        with pytest.raises(pkv.PagedKVError):
            graph.replay(5, stream=stream)
        with pytest.raises(pkv.PagedKVError):
            graph.replay(0, stream=stream)
    finally:
        graph.close()
        ds.free()


def test_back_to_back_replays_with_changing_counts():
    """Replays enqueued without a wait between them, the second with one real
    request fewer (the plan node's arguments are rewritten between the two
    launches): each runs with its own count.  The new row of the request that
    only the first replay treats as real must hold its K/V afterwards, and the
    outputs are the second replay's, bit-identical to the eager padded batch."""
    w = decode_workload(91, 1)
    log(f"back-to-back replays: {w.summary()}")
    ds = device_step(w)
    stream = torch.cuda.Stream()
    ref = P.oracle_for(w)
    rows = ref["meta"]["out_loc"]
    n = w.num_reqs
    graph = pkv.DecodeGraph(ds.pool, ds.page_table, ds.batch, ds.alloc_rows, ds.q, ds.o, ds.k_new, ds.v_new,
                            ds.meta, ds.workspace, w.sm_scale, int(w.dummy_table_row), [n], stream)
    try:
        want = eager_padded(ds, w, n - 1, n, stream)
        for rep in range(5):
            write_real(ds, w, n)
            last = torch.as_tensor([int(rows[n - 1])], device=ds.device)
            ds.k_pool[last] = 0
            ds.v_pool[last] = 0
            ds.o.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay(n, stream=stream)
            graph.replay(n - 1, stream=stream)
            stream.synchronize()
            k, v = ds.pool_rows_bits([int(rows[n - 1])])
            assert np.array_equal(k[0], w.k_new[n - 1]) and np.array_equal(v[0], w.v_new[n - 1]), \
                f"rep {rep}: the first replay did not run with all {n} requests"
            got = ds.o[:n - 1]
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"rep {rep}: outputs"
            assert ds.status() == 0
    finally:
        graph.close()
        ds.free()
