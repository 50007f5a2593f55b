"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small variants of the five workloads are checked on every output; the
full-size workloads (the sizes the benchmark times, in the same launch
configuration) are checked bit-exactly on metadata and store and on sampled
attention outputs.  Every case also checks that no pool row outside the new
tokens' rows and the dummy page changed (whole pool, wherever a copy of it
fits next to it) and reads the plan back to check that its work lists cover
every (request, KV head, key) of the decode and every (request, new token) of
the extend exactly once.  Planted-spike cases pin the gather at specific
positions (first row, last row, tile, page and decode-run boundaries), where a
dropped or shifted key would otherwise hide in the small N(0,1) outputs of
long contexts.
"""
import functools

import numpy as np
import pytest
import torch

from workloads import RequestSpec, build_workload, configs
import paged_kv_attention_08_amd as pkv
from tests.gpu_harness import DeviceStep, log
from tests import parity_checks as P

pytestmark = pytest.mark.gpu


WHOLE_POOL_MAX_ROWS = 1 << 22  # a copy of pools up to 16 GiB (K + V) is taken for the diff


def run_case(w, decode_requests=None, extend_tokens=None, label="", fused_store=False):
    log(f"case {label}: {w.summary()}")
    ds = DeviceStep(w)
    before = ds.snapshot_pool() if w.num_pool_rows <= WHOLE_POOL_MAX_ROWS else None
    log("  device step" + (" (metadata and store in one call)" if fused_store else ""))
    ds.run(fused_store=fused_store)
    torch.cuda.synchronize()
    log("  device step done")
    assert ds.status() == 0, f"device status bits {ds.status():#x}"
    ref = P.oracle_for(w, decode_requests, extend_tokens)
    P.check_metadata(ds, ref, w)
    P.check_store(ds, ref, w)
    if before is not None:
        n_changed = P.check_pool_unchanged_elsewhere(ds, before, P.allowed_changed_rows(ref, w))
        del before
        torch.cuda.empty_cache()
        log(f"  whole pool: {n_changed} rows changed, all new-token or dummy rows")
    plan, view = ds.plan_host()
    cover = P.check_plan_coverage(plan, view, w)
    log(f"  plan coverage ok {cover}")
    P.real_outputs_finite(ds, w)
    stats = P.check_attention(ds, ref["out"], w, label)
    log(f"  ok {stats}")
    return ds, ref, stats


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_wide_scores(cfg):
    """q and K at 3 times N(0, 1): scores with a standard deviation near 9, so
    each softmax row sits on a few keys and the rounding of the score scaling
    shows (tests/test_parity_sensitivity.py: the bar passes fp32 scaling and
    fails q * scale rounded to bf16 at this spread)."""
    w = P.widen_scores(configs.small(cfg), 3.0)
    run_case(w, label=f"wide-scores-{cfg}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_small_config(cfg):
    w = configs.small(cfg)
    ds, _, _ = run_case(w, label=f"small{cfg}")
    ds.free()


def full_samples(cfg, w):
    """Decode requests and extend tokens of a full-size workload that the
    oracle checks one by one (None: all of them)."""
    dec = None
    if w.num_decode > 64:
        rng = np.random.default_rng(cfg)
        dec = sorted(set(rng.choice(w.num_decode, 48, replace=False).tolist()) | {0, w.num_decode - 1})
    elif cfg == 4:
        dec = [0, 7, 15, 31]
    ext = P.sample_tokens(w, per_request=6, seed=cfg) if w.num_decode < w.num_reqs else None
    return dec, ext


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_config(cfg):
    w = configs.FULL[cfg]()
    dec, ext = full_samples(cfg, w)
    ds, _, _ = run_case(w, decode_requests=dec, extend_tokens=ext, label=f"full{cfg}")
    ds.free()


def _bf16(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _plant(w, spikes, seed=17):
    """For each request i, make every key position in spikes[i] dominate all
    queries of the request with one score (every query is a vector u, every
    planted K row is 4u in all KV heads) and give each planted key a one-hot V
    at its own dimension.  A token that sees n of them must return 1/n at each
    of their dimensions and about 0 elsewhere.  Returns {i: [(position, dim)]}."""
    d = w.head_dim
    row_of_cached = {int(r): n for n, r in enumerate(w.cached_rows)}
    starts = P.token_starts(w)
    rng = np.random.default_rng(seed)
    planted = {}
    owner = {}  # a radix-shared cached row is planted only by the first request that reads it
    for i in sorted(spikes):
        for j in range(int(w.cached_len[i])):
            owner.setdefault(int(w.page_table[w.table_idx[i], j]), i)
    for i, positions in spikes.items():
        c = int(w.cached_len[i])
        positions = sorted(set(int(j) for j in positions
                               if j >= c or owner[int(w.page_table[w.table_idx[i], j])] == i))
        assert len(positions) <= d, "one dimension per planted key"
        t0, t1 = starts[i], starts[i + 1]
        c = int(w.cached_len[i])
        u = rng.normal(size=d).astype(np.float32)
        w.q[t0:t1, :, :] = _bf16(u)[None, None, :]
        kb = _bf16(u * 4)
        dims = rng.permutation(d)[:len(positions)]
        for j, hot in zip(positions, dims):
            onehot = np.zeros(d, dtype=np.uint16)
            onehot[hot] = 0x3F80  # 1.0
            if j < c:
                n = row_of_cached[int(w.page_table[w.table_idx[i], j])]
                w.k_cached[n, :, :] = kb[None, :]
                w.v_cached[n, :, :] = onehot[None, :]
            else:
                t = t0 + (j - c)
                w.k_new[t, :, :] = kb[None, :]
                w.v_new[t, :, :] = onehot[None, :]
        planted[i] = list(zip(positions, (int(x) for x in dims)))
    return planted


def _check_spikes(ds, w, planted):
    """Every real token returns 1/n at the dimensions of the n planted keys it
    sees (to a quarter of 1/n) and no more than that error elsewhere."""
    starts = P.token_starts(w)
    checked = 0
    for i, keys in planted.items():
        c = int(w.cached_len[i])
        toks = list(range(starts[i], starts[i + 1]))
        got_all = ds.output_f64(toks)
        for k, t in enumerate(toks):
            pos = c + (t - starts[i])
            vis = [dim for j, dim in keys if j <= pos]
            if not vis:
                continue
            want = np.zeros(w.head_dim)
            want[vis] = 1.0 / len(vis)
            err = np.abs(got_all[k] - want[None, :]).max()
            assert err < 0.25 / len(vis), (f"request {i} token {t}: {len(vis)} planted keys visible, "
                                           f"max err {err:.3e}")
            checked += 1
    return checked


def _run_boundary_keys(w, view):
    """Key positions where one decode run's share of the flat tile order ends
    and the next begins, inside each decode request, with the share `per` the
    plan derives from the lengths (run r takes flat tiles [r per, (r+1) per))."""
    K, HG, runs = view["decode_tile_keys"], view["decode_group_heads"], view["decode_runs"]
    Hg = w.num_kv_heads // HG
    n = [-(-int(w.device_len[i]) // K) for i in range(w.num_decode)]
    seg = np.concatenate([[0], np.cumsum(n)]) * Hg
    total = int(seg[-1])
    per = max(1, -(-total // runs))
    out = {i: [] for i in range(w.num_decode)}
    for f in range(per, total, per):
        i = int(np.searchsorted(seg, f, side="right") - 1)
        local = f - int(seg[i])
        kti = local % n[i]
        if kti:  # a boundary inside the request's keys (not at a segment start)
            out[i] += [K * kti - 1, K * kti]
    return out, per


def _spike_case(kind):
    if kind == "decode":
        w = configs.serving_decode(seed=31, real=12, padded_to=16, lo=1500, hi=2600, num_pool_rows=1 << 16)
    elif kind == "extend":
        w = configs.extend_radix(seed=32, nreq=3, prefix=256, tail_hi=200, chunk=300, num_pool_rows=1 << 14)
    elif kind == "page64":
        w = configs.mixed_page64(seed=33, ndec=8, dec_lo=600, dec_hi=900, next_=2, pre_hi=300, new_tokens=130,
                                 num_pool_rows=64 * 128)
    elif kind == "long_runs":
        # the long-decode shape: 64 query / 8 KV heads, contexts 16K-32K; 16
        # requests, so each one spans about 16 decode runs
        w = configs.long_decode(seed=34, batch=16, num_pool_rows=1 << 19)
    else:  # "page64_runs": page size 64 at the mixed batch's decode lengths (1K-8K) plus extend requests
        w = configs.mixed_page64(seed=35, ndec=16, next_=2, new_tokens=160, num_pool_rows=1 << 18)
    return w


@pytest.mark.parametrize("kind", ["decode", "extend", "page64", "long_runs", "page64_runs"])
def test_planted_spikes(kind):
    w = _spike_case(kind)
    view = pkv.plan_view(w.num_reqs, w.num_tokens, w.num_qo_heads, w.num_kv_heads)
    bounds, per = _run_boundary_keys(w, view)
    s = w.page_size
    spikes = {}
    for i in range(w.num_reqs):
        if w.is_padding[i]:
            continue
        dl, c = int(w.device_len[i]), int(w.cached_len[i])
        pos = {0, dl - 1, min(31, dl - 1), min(32, dl - 1), min(63, dl - 1), min(64, dl - 1)}
        if s > 1:  # page boundaries near the middle
            m = max(1, (dl // 2) // s) * s
            pos |= {m - 1, min(m, dl - 1)}
        if i >= w.num_decode:  # last cached and first new key of an extend request
            pos |= {max(c - 1, 0), c}
        pos |= set(bounds.get(i, []))
        spikes[i] = sorted(pos)
    planted = _plant(w, spikes)
    ds, ref, _ = run_case(w, label=f"spike-{kind}")
    plan, _ = ds.plan_host()
    hdr, _, _ = P.plan_arrays(plan, view, w.num_reqs)
    if w.num_decode:
        assert int(hdr[1]) == per, "spikes were placed for another decode share"
    else:
        assert not any(bounds.values())
    n_bounds = sum(len(b) for b in bounds.values()) // 2
    checked = _check_spikes(ds, w, planted)
    log(f"  {checked} tokens checked, {n_bounds} run boundaries inside requests")
    if kind in ("long_runs", "page64_runs"):
        assert n_bounds >= 8 * w.num_decode
    ds.free()


@pytest.mark.parametrize("which", ["small5", "full3"])
def test_attention_repeated_on_one_plan(which):
    """The attention calls run again on the same metadata (as every layer of a
    model does) give the same results each time: state they keep in the plan
    between workgroups is back at its start when a call ends."""
    if which == "small5":
        w, ext = configs.small(5), None
    else:
        w = configs.FULL[3]()
        ext = P.sample_tokens(w, per_request=4, seed=33)
    ds, ref, _ = run_case(w, extend_tokens=ext, label=f"repeat {which}")
    for r in range(3):
        ds.o.fill_(float("nan"))
        if w.num_decode:
            ds.decode()
        ds.extend()
        torch.cuda.synchronize()
        assert ds.status() == 0
        P.real_outputs_finite(ds, w)
        stats = P.check_attention(ds, ref["out"], w, f"repeat {which} call {r + 2}")
        log(f"  call {r + 2} ok {stats}")
    ds.free()


@functools.lru_cache(maxsize=1)
def _edge_workloads():
    """The edge-case batches (built once per session; the tests do not modify them)."""
    cases = []
    # every request has a single key: the output is that key's V, exactly
    cases.append(("single_key", build_workload("single_key", 41, [RequestSpec(0, 1) for _ in range(5)],
                                               num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=1,
                                               num_pool_rows=256, num_decode=5)))
    # pure prefill (cached_len 0), MHA (G = 1)
    cases.append(("prefill_mha", build_workload("prefill_mha", 42, [RequestSpec(0, 77), RequestSpec(0, 130)],
                                                num_qo_heads=8, num_kv_heads=8, head_dim=128, page_size=1,
                                                num_pool_rows=1024, num_decode=0)))
    # G = 16 (one KV head), decode and extend mixed
    cases.append(("group16", build_workload("group16", 43, [RequestSpec(300, 301), RequestSpec(5, 6),
                                                            RequestSpec(40, 111)],
                                            num_qo_heads=16, num_kv_heads=1, head_dim=128, page_size=1,
                                            num_pool_rows=1024, num_decode=2)))
    # G = 2 and odd G = 3
    cases.append(("group2", build_workload("group2", 44, [RequestSpec(100, 101), RequestSpec(33, 97)],
                                           num_qo_heads=8, num_kv_heads=4, head_dim=128, page_size=1,
                                           num_pool_rows=1024, num_decode=1)))
    cases.append(("group3", build_workload("group3", 45, [RequestSpec(70, 71), RequestSpec(12, 60)],
                                           num_qo_heads=6, num_kv_heads=2, head_dim=128, page_size=1,
                                           num_pool_rows=1024, num_decode=1)))
    # KV head counts whose decode runs read 2 heads (6 KV heads) and 1 head (3 KV heads) at a time
    cases.append(("kv6", build_workload("kv6", 56, [RequestSpec(700, 701), RequestSpec(64, 65), RequestSpec(2, 3),
                                                    RequestSpec(10, 90)],
                                        num_qo_heads=12, num_kv_heads=6, head_dim=128, page_size=1,
                                        num_pool_rows=2048, num_decode=3)))
    cases.append(("kv3", build_workload("kv3", 57, [RequestSpec(500, 501), RequestSpec(31, 32), RequestSpec(3, 40)],
                                        num_qo_heads=12, num_kv_heads=3, head_dim=128, page_size=1,
                                        num_pool_rows=2048, num_decode=2)))
    # a pool of 4 GiB per K and V: extend gathers take 64-bit row offsets
    cases.append(("wide_pool", build_workload("wide_pool", 58, [RequestSpec(900, 901), RequestSpec(300, 470),
                                                                RequestSpec(0, 129)],
                                              num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=1,
                                              num_pool_rows=(1 << 21) + 64, num_decode=1)))
    # other page sizes with partial pages on both ends
    for s in (2, 16, 32):
        cases.append((f"page{s}", build_workload(f"page{s}", 46 + s, [RequestSpec(5 * s + 3, 5 * s + 4),
                                                                      RequestSpec(s - 1, 3 * s + 2),
                                                                      RequestSpec(0, 1, padding=True)],
                                                 num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=s,
                                                 num_pool_rows=64 * s, num_decode=1)))
    # pages in allocation order (a fresh pool's free list) instead of a random order
    cases.append(("seq_pages", configs.extend_radix(seed=59, nreq=3, prefix=96, tail_hi=70, chunk=83,
                                                    num_pool_rows=1 << 13, page_order="sequential")))
    cases.append(("seq_pages64", configs.mixed_page64(seed=61, ndec=6, dec_lo=1, dec_hi=300, next_=3, pre_hi=200,
                                                      new_tokens=150, num_pool_rows=64 * 64,
                                                      page_order="sequential")))
    # batches at the size where build_attn_metadata stops mapping the tokens inside its
    # plan launch (1024 requests: the LDS copy of the running totals) and launches a
    # kernel for them, and at the earlier threshold of 512 new tokens
    for nreq in (512, 513, 1024, 1025):
        lens = [(37 * k) % 300 + 1 for k in range(nreq)]
        reqs = [RequestSpec(l, l + 1) for l in lens]
        cases.append((f"meta{nreq}", build_workload(f"meta{nreq}", 62 + nreq % 2, reqs, num_qo_heads=32,
                                                    num_kv_heads=8, head_dim=128, page_size=1,
                                                    num_pool_rows=1 << 18, num_decode=nreq)))
    # the largest query-head group (16 per KV head: the largest decode workspace) at long-decode lengths
    cases.append(("group16_long", build_workload("group16_long", 64, [RequestSpec(17000, 17001),
                                                                      RequestSpec(30001, 30002),
                                                                      RequestSpec(20000, 20004)],
                                                 num_qo_heads=128, num_kv_heads=8, head_dim=128, page_size=1,
                                                 num_pool_rows=1 << 17, num_decode=2)))
    # 4096 decode requests: past the plan kernel's LDS copy of the running totals (1024 requests)
    lens = [(53 * k) % 97 + 1 for k in range(4096)]
    cases.append(("batch4096", build_workload("batch4096", 65, [RequestSpec(l, l + 1) for l in lens],
                                              num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=1,
                                              num_pool_rows=1 << 19, num_decode=4096)))
    # extend items of 1 to 9 key tiles of 64 (the extend loop runs whole groups of four tiles, then up to
    # three more one by one; every count of groups and leftover tiles), and a prefill whose items end
    # at 64, 128, 192, 256 and 300 keys
    spans = [(0, 1), (63, 1), (64, 1), (127, 2), (190, 3), (256, 1), (320, 20), (400, 30), (447, 65), (520, 10),
             (0, 300)]
    cases.append(("key_tiles", build_workload("key_tiles", 66, [RequestSpec(c, c + e) for c, e in spans],
                                              num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=1,
                                              num_pool_rows=1 << 14, num_decode=0)))
    # one long decode request spread over many splits, width exactly its length rounded to 32
    cases.append(("long_single", build_workload("long_single", 50, [RequestSpec(20000, 20001)],
                                                num_qo_heads=64, num_kv_heads=8, head_dim=128, page_size=1,
                                                num_pool_rows=1 << 16, num_decode=1)))
    return cases


@pytest.mark.parametrize("name", [n for n, _ in _edge_workloads()])
def test_edge_case(name):
    w = dict(_edge_workloads())[name]
    ds, ref, _ = run_case(w, label=name)
    if name == "single_key":
        # one key: the output must be that key's V bit for bit (p = 1, l = 1)
        got = ds.o.view(torch.int16).cpu().numpy().view(np.uint16)
        group = w.num_qo_heads // w.num_kv_heads
        for t in range(w.num_tokens):
            for h in range(w.num_qo_heads):
                assert np.array_equal(got[t, h], w.v_new[t, h // group])
    ds.free()


def test_empty_batch():
    w = build_workload("empty", 60, [], num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=1,
                       num_pool_rows=64, num_decode=0)
    log("case empty batch")
    ds = DeviceStep(w)
    ds.run()
    torch.cuda.synchronize()
    assert ds.status() == 0
    assert int(ds.meta.qo_indptr[0].item()) == 0 and int(ds.meta.kv_indptr[0].item()) == 0
    ds.free()


FUSED_CASES = ["small1", "small2", "small3", "small4", "small5", "full1", "full2", "full3", "full5", "single_key",
               "group16", "kv3", "page2", "page16", "page32", "seq_pages64", "meta512", "meta513", "meta1024",
               "meta1025", "batch4096"]


@pytest.mark.parametrize("name", FUSED_CASES)
def test_metadata_and_store_in_one_call(name):
    """build_attn_metadata_store gives what build_attn_metadata + kv_store give:
    the same bit-exact metadata, stored rows and untouched pool, and outputs
    within the bar (one launch up to 1024 requests, any number of new tokens:
    meta1024, full3; two above: meta1025, batch4096)."""
    ext = None
    if name.startswith("small"):
        w = configs.small(int(name[5:]))
    elif name.startswith("full"):
        w = configs.FULL[int(name[4:])]()
        _, ext = full_samples(int(name[4:]), w)  # every decode request, sampled extend tokens
    else:
        w = dict(_edge_workloads())[name]
    ds, _, _ = run_case(w, extend_tokens=ext, label=f"fused {name}", fused_store=True)
    ds.free()
