"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin is a plain function that raises AssertionError (or any exception) on
failure, so that ``test_oracle.py`` can run all of them against the real oracle
and, in the mutation test, against deliberately broken variants of it.

Sources of truth used here, none of which re-types an oracle formula:
* torch's scaled_dot_product_attention in float64 on the CPU (a library
  routine) with an explicit bottom-right boolean mask and enable_gqa;
* scipy.special.softmax (a library routine);
* closed forms: one key gives that key's V; equal V rows give that row; q = 0
  or equal K rows give the mean of V; a dominant key gives its V; scores
  (ln 3, 0) give weights (3/4, 1/4);
* invariants: a permuted physical layout, private copies of a shared prefix,
  padding requests, and splitting a chunk in two leave real outputs unchanged;
* numpy.cumsum / arange for the metadata's running totals and positions; an
  independent page-list reconstruction of every request's physical rows;
* the source pages' printed KV-size estimate (tests/golden).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch

import oracle.pagedkv_oracle as O
from oracle.run import initial_pool, reference_step
from workloads import RequestSpec, build_workload, float32_to_bf16_bits
from workloads import configs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# helpers that build inputs by hand (no oracle arithmetic)
# ----------------------------------------------------------------------------

def tiny(seed=3, page_size=1, hq=4, hkv=2, d=16, reqs=None, pool_rows=256, num_decode=None):
    reqs = reqs or [RequestSpec(5, 6), RequestSpec(0, 7), RequestSpec(9, 13), RequestSpec(3, 4)]
    nd = num_decode if num_decode is not None else 0
    return build_workload("tiny", seed, reqs, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d,
                          page_size=page_size, num_pool_rows=pool_rows, num_decode=nd)


def logical_kv(w, i):
    """Request i's K and V in logical token order, built directly from the
    generator's arrays: cached tokens via the pre-batch page table and the
    cached-row values, new tokens from k_new / v_new in batch order."""
    row_to_idx = {int(r): n for n, r in enumerate(w.cached_rows)}
    c, dl = int(w.cached_len[i]), int(w.device_len[i])
    t0 = int((w.device_len[:i].astype(np.int64) - w.cached_len[:i]).sum())
    K, V = [], []
    for j in range(dl):
        if j < c:
            n = row_to_idx[int(w.page_table[w.table_idx[i], j])]
            K.append(w.k_cached[n]); V.append(w.v_cached[n])
        else:
            K.append(w.k_new[t0 + j - c]); V.append(w.v_new[t0 + j - c])
    return O.widen_bf16(np.stack(K)), O.widen_bf16(np.stack(V)), t0


def sdpa_reference(w, i):
    """torch SDPA (float64, CPU) over request i's logical K/V with a
    bottom-right causal mask and GQA head sharing."""
    K, V, t0 = logical_kv(w, i)
    c, dl = int(w.cached_len[i]), int(w.device_len[i])
    n = dl - c
    q = O.widen_bf16(w.q[t0:t0 + n])                         # [n, Hq, d]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]          # [1, Hq, n, d]
    kt = torch.from_numpy(K).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(V).permute(1, 0, 2)[None].contiguous()
    mask = torch.arange(dl)[None, :] <= (c + torch.arange(n))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=w.sm_scale,
                                                         enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy(), t0


def run_all(w):
    return reference_step(w)


def permuted(w, seed=11):
    """Same batch, physical pages relabelled by a random permutation that keeps
    the dummy page and the poison page in place."""
    s = w.page_size
    P = w.num_pool_rows // s
    rng = np.random.default_rng(seed)
    perm = np.arange(P)
    perm[1:P - 1] = rng.permutation(np.arange(1, P - 1))

    def remap(rows):
        rows = np.asarray(rows, dtype=np.int64)
        return perm[rows // s] * s + rows % s

    pt = w.page_table.astype(np.int64)
    new = dict(w.__dict__)
    new["page_table"] = remap(pt).astype(np.int32)
    new["alloc_rows"] = remap(w.alloc_rows).astype(np.int32)
    new["cached_rows"] = remap(w.cached_rows)
    return type(w)(**new), remap


# ----------------------------------------------------------------------------
# attention pins
# ----------------------------------------------------------------------------

def pin_sdpa_library():
    for w in (tiny(), tiny(page_size=4, seed=5), tiny(hq=6, hkv=2, seed=8),
              tiny(hq=3, hkv=3, seed=9, reqs=[RequestSpec(0, 5), RequestSpec(7, 8)])):
        res = run_all(w)
        for i in range(w.num_reqs):
            ref, t0 = sdpa_reference(w, i)
            for t in range(ref.shape[0]):
                np.testing.assert_allclose(res["out"][t0 + t], ref[t], rtol=0, atol=1e-12)


def pin_softmax_library():
    rng = np.random.default_rng(0)
    for n in (1, 2, 7, 300):
        s = rng.normal(size=n) * 10
        np.testing.assert_allclose(O.softmax(s), scipy.special.softmax(s), rtol=1e-13, atol=1e-300)


def pin_permutation_invariance():
    mixed = tiny(page_size=4, seed=14, num_decode=2, reqs=[RequestSpec(9, 10), RequestSpec(4, 5),
                 RequestSpec(6, 19), RequestSpec(0, 11), RequestSpec(0, 1, padding=True)])
    for w in (tiny(), tiny(page_size=4, seed=4), mixed):
        a = run_all(w)
        wp, remap = permuted(w)
        b = run_all(wp)
        assert a["out"].keys() == b["out"].keys()
        for t in a["out"]:
            assert np.array_equal(a["out"][t], b["out"][t])
        assert np.array_equal(remap(a["meta"]["out_loc"]), b["meta"]["out_loc"])


def pin_padding_invariance():
    w = configs.serving_decode(seed=5, real=6, padded_to=9, lo=1, hi=90, num_pool_rows=1024, num_qo_heads=16)
    pad = np.nonzero(w.is_padding)[0]
    assert pad.size and np.all(pad == np.arange(w.num_reqs - pad.size, w.num_reqs))
    real = w.num_reqs - pad.size
    t_real = int((w.device_len[:real].astype(np.int64) - w.cached_len[:real]).sum())
    n_alloc_real = len(w.alloc_rows) - pad.size
    new = dict(w.__dict__)
    for k in ("table_idx", "cached_len", "device_len", "is_padding"):
        new[k] = getattr(w, k)[:real]
    for k in ("q", "k_new", "v_new"):
        new[k] = getattr(w, k)[:t_real]
    new["alloc_rows"] = w.alloc_rows[:n_alloc_real]
    w2 = type(w)(**new)
    a, b = run_all(w), run_all(w2)
    for t in range(t_real):
        assert np.array_equal(a["out"][t], b["out"][t])
    # padded tokens only touch the dummy page
    pa, pb = a["pool"], b["pool"]
    rows = set(pa.written_rows()) | set(pb.written_rows())
    for r in rows:
        if r in w.dummy_rows:
            continue
        ka, kb = pa.row_bits(r), pb.row_bits(r)
        assert ka is not None and kb is not None
        assert np.array_equal(ka[0], kb[0]) and np.array_equal(ka[1], kb[1])
    assert all(int(x) in w.dummy_rows for x in a["meta"]["out_loc"][t_real:])


def pin_prefix_sharing():
    shared = 40
    w = configs.extend_radix(seed=2, nreq=3, prefix=shared, tail_hi=12, chunk=9, num_pool_rows=512)
    a = run_all(w)
    # give every request a private copy of the shared prefix at fresh rows
    used = set(int(r) for r in w.cached_rows) | set(int(r) for r in w.alloc_rows)
    free = [r for r in range(1, w.num_pool_rows - 1) if r not in used]
    pt = w.page_table.copy()
    rows = list(w.cached_rows)
    kc, vc = list(w.k_cached), list(w.v_cached)
    idx = {int(r): n for n, r in enumerate(w.cached_rows)}
    cur = 0
    for i in range(1, w.num_reqs):           # request 0 keeps the original rows
        r = w.table_idx[i]
        for j in range(shared):
            old = int(pt[r, j])
            new_row = free[cur]; cur += 1
            pt[r, j] = new_row
            rows.append(new_row); kc.append(w.k_cached[idx[old]]); vc.append(w.v_cached[idx[old]])
    new = dict(w.__dict__)
    new.update(page_table=pt, cached_rows=np.array(rows, dtype=np.int64), k_cached=np.stack(kc),
               v_cached=np.stack(vc))
    b = run_all(type(w)(**new))
    for t in a["out"]:
        assert np.array_equal(a["out"][t], b["out"][t])


def pin_chunk_split():
    for s in (1, 4):
        w = tiny(seed=21, page_size=s, reqs=[RequestSpec(6, 17), RequestSpec(0, 9)], pool_rows=256)
        whole = run_all(w)
        cut = [4, 5]                                   # first part of each request's chunk
        # part 1: device_len = cached + cut
        new1 = dict(w.__dict__)
        dl1 = w.cached_len + np.array(cut, dtype=np.int32)
        tok = []
        start = 0
        for i in range(w.num_reqs):
            ext = int(w.device_len[i] - w.cached_len[i])
            tok.append((start, ext)); start += ext
        sel1 = np.concatenate([np.arange(a, a + c) for (a, _), c in zip(tok, cut)])
        sel2 = np.concatenate([np.arange(a + c, a + e) for (a, e), c in zip(tok, cut)])
        # pages for part 1 / part 2, in request order
        alloc1, alloc2 = [], []
        cur = 0
        for i in range(w.num_reqs):
            n_all = -(-int(w.device_len[i]) // s) - (-(-int(w.cached_len[i]) // s))
            n1 = -(-int(dl1[i]) // s) - (-(-int(w.cached_len[i]) // s))
            alloc1 += list(w.alloc_rows[cur:cur + n1]); alloc2 += list(w.alloc_rows[cur + n1:cur + n_all])
            cur += n_all
        new1.update(device_len=dl1, q=w.q[sel1], k_new=w.k_new[sel1], v_new=w.v_new[sel1],
                    alloc_rows=np.array(alloc1, dtype=np.int32))
        w1 = type(w)(**new1)
        r1 = run_all(w1)
        # part 2 continues from part 1's page table and pool
        meta2 = O.build_metadata(r1["meta"]["page_table"], w.table_idx, dl1, w.device_len,
                                 np.array(alloc2, dtype=np.int32), s)
        pool2 = O.store_kv(r1["pool"], w.k_new[sel2], w.v_new[sel2], meta2["out_loc"])
        out2 = O.paged_attention(pool2, meta2["page_table"], w.table_idx, dl1, w.device_len, w.q[sel2],
                                 w.num_kv_heads, w.sm_scale)
        assert np.array_equal(meta2["page_table"], whole["meta"]["page_table"])
        for n, t in enumerate(sel1):
            assert np.array_equal(r1["out"][n], whole["out"][int(t)])
        for n, t in enumerate(sel2):
            assert np.array_equal(out2[n], whole["out"][int(t)])


def _single_request_pool(K_bits, V_bits, d=8, hkv=1):
    n = K_bits.shape[0]
    pool = O.KVPool(64, hkv, d)
    rows = list(range(10, 10 + n))
    pool.load(rows, K_bits.reshape(n, hkv, d), V_bits.reshape(n, hkv, d))
    pt = np.zeros((1, 64), dtype=np.int32)
    pt[0, :n] = rows
    return pool, pt


def _attend_one(q_bits, K_bits, V_bits, scale):
    """One decode query (chunk offset 0) over all n keys through the oracle."""
    n = K_bits.shape[0]
    pool, pt = _single_request_pool(K_bits, V_bits, d=K_bits.shape[-1])
    out = O.paged_attention(pool, pt, np.array([0]), np.array([n - 1]), np.array([n]), q_bits[None, None, :],
                            1, scale)
    return out[0][0]


def pin_closed_forms():
    rng = np.random.default_rng(1)
    bf = lambda x: float32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    d = 8
    # one key -> that V, exactly
    K = bf(rng.normal(size=(1, d))); V = bf(rng.normal(size=(1, d))); q = bf(rng.normal(size=d))
    assert np.array_equal(_attend_one(q, K, V, 0.3), O.widen_bf16(V[0]))
    # equal V rows -> that row
    n = 37
    K = bf(rng.normal(size=(n, d))); row = rng.normal(size=d); V = bf(np.tile(row, (n, 1)))
    np.testing.assert_allclose(_attend_one(bf(rng.normal(size=d)), K, V, 0.5), O.widen_bf16(V[0]),
                               rtol=1e-14, atol=1e-15)
    # q = 0 -> mean of V ; equal K rows -> mean of V
    V = bf(rng.normal(size=(n, d)))
    mean = O.widen_bf16(V).mean(axis=0)
    np.testing.assert_allclose(_attend_one(bf(np.zeros(d)), bf(rng.normal(size=(n, d))), V, 1.0), mean,
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(_attend_one(bf(rng.normal(size=d)), bf(np.tile(rng.normal(size=d), (n, 1))), V,
                                           1.0), mean, rtol=0, atol=1e-14)
    # scores (ln 3, 0) -> weights (3/4, 1/4)
    e0 = np.zeros(d); e0[0] = 1.0
    K = bf(np.stack([e0, np.zeros(d)])); V = bf(rng.normal(size=(2, d)))
    Vw = O.widen_bf16(V)
    np.testing.assert_allclose(_attend_one(bf(e0), K, V, math.log(3.0)), 0.75 * Vw[0] + 0.25 * Vw[1],
                               rtol=1e-14, atol=1e-15)
    # a dominant key (score ~ 2000, far past exp overflow without the max shift) -> its V
    n = 50
    K = bf(rng.normal(size=(n, d)) * 0.1)
    star = 23
    K[star] = bf(np.full(d, 16.0))
    q = bf(np.full(d, 16.0))
    V = bf(rng.normal(size=(n, d)))
    got = _attend_one(q, K, V, 1.0)
    np.testing.assert_allclose(got, O.widen_bf16(V[star]), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# metadata and store pins
# ----------------------------------------------------------------------------

def _meta_workloads():
    return [tiny(), tiny(page_size=4, seed=6), tiny(page_size=8, seed=12, reqs=[RequestSpec(13, 14),
            RequestSpec(16, 40), RequestSpec(0, 1, padding=True), RequestSpec(0, 1, padding=True)]),
            configs.small(5, seed=4), configs.small(2, seed=9)]


def pin_metadata_running_totals():
    for w in _meta_workloads():
        m = reference_step(w, attention=False)["meta"]
        ext = w.device_len.astype(np.int64) - w.cached_len
        assert np.array_equal(m["qo_indptr"], np.concatenate([[0], np.cumsum(ext)]))
        assert np.array_equal(m["kv_indptr"], np.concatenate([[0], np.cumsum(w.device_len.astype(np.int64))]))
        pos = np.concatenate([np.arange(c, dl) for c, dl in zip(w.cached_len, w.device_len)])
        assert np.array_equal(m["positions"], pos)
        # each request's last new token is the one at position device_len - 1
        owner = np.repeat(np.arange(w.num_reqs), ext)
        for i in range(w.num_reqs):
            t = m["last_indices"][i]
            assert owner[t] == i and m["positions"][t] == w.device_len[i] - 1


def pin_metadata_page_list():
    """Rebuild every request's physical rows from its page list."""
    for w in _meta_workloads():
        m = reference_step(w, attention=False)["meta"]
        s = w.page_size
        pt = m["page_table"]
        cur = 0
        changed = np.zeros(pt.shape, dtype=bool)
        for i in range(w.num_reqs):
            r = w.table_idx[i]
            c, dl = int(w.cached_len[i]), int(w.device_len[i])
            old_pages = [int(w.page_table[r, p * s]) // s for p in range(-(-c // s))]
            k_new = -(-dl // s) - len(old_pages)
            new_pages = [int(x) // s for x in w.alloc_rows[cur:cur + k_new]]
            cur += k_new
            pages = old_pages + new_pages
            expect = np.array([pages[j // s] * s + j % s for j in range(dl)], dtype=np.int64)
            assert np.array_equal(pt[r, :dl].astype(np.int64), expect), (i, w.name)
            changed[r, c:dl] = True
        assert cur == len(w.alloc_rows)
        assert np.array_equal(pt[~changed], w.page_table[~changed])
        owner = np.repeat(np.arange(w.num_reqs), w.device_len.astype(np.int64) - w.cached_len)
        for t, row in enumerate(m["out_loc"]):
            i = owner[t]
            assert row == pt[w.table_idx[i], m["positions"][t]]
        # new rows of real requests are distinct, outside dummy/poison pages, not cached rows
        real_rows = [int(m["out_loc"][t]) for t in range(len(owner)) if not w.is_padding[owner[t]]]
        assert len(set(real_rows)) == len(real_rows)
        assert not set(real_rows) & (set(w.dummy_rows) | set(w.poison_rows) | set(int(x) for x in w.cached_rows))
        if s == 1:
            assert np.array_equal(m["out_loc"], w.alloc_rows)


def pin_store():
    w = tiny(seed=31)
    res = reference_step(w, attention=False)
    before, after = initial_pool(w), res["pool"]
    out_loc = [int(x) for x in res["meta"]["out_loc"]]
    for t, row in enumerate(out_loc):
        kb, vb = after.row_bits(row)
        assert np.array_equal(kb, w.k_new[t]) and np.array_equal(vb, w.v_new[t])
    for row in before.written_rows():
        if row not in out_loc:
            assert np.array_equal(after.row_bits(row)[0], before.row_bits(row)[0])
            assert np.array_equal(after.row_bits(row)[1], before.row_bits(row)[1])
    # two writes to one row (padding on the dummy page): the later write wins
    pool = O.KVPool(8, 1, 4)
    a = np.arange(4, dtype=np.uint16).reshape(1, 1, 4)
    b = (np.arange(4, dtype=np.uint16) + 100).reshape(1, 1, 4)
    p2 = O.store_kv(pool, np.concatenate([a, b]), np.concatenate([b, a]), np.array([0, 0]))
    assert np.array_equal(p2.row_bits(0)[0], b[0]) and np.array_equal(p2.row_bits(0)[1], a[0])


def pin_byte_model():
    with open(os.path.join(GOLDEN, "kv_bytes_deep_dive_6_1.json")) as f:
        g = json.load(f)
    one = O.kv_bytes(g["num_layers"], g["num_kv_heads"], g["head_dim"], g["num_tokens"], g["dtype_bytes"])
    assert one == g["exact_bytes_one_request"]
    assert round(one / 2 ** 30) == g["quoted_gb_one_request"]
    assert round(100 * one / 1e9, -2) == g["quoted_gb_hundred_requests"]
    # hand-worked decode bytes: one key, 8 KV heads, d 128, 32 query heads, page size 1:
    # K+V 2*8*128*2 = 4096 B, one 4-byte entry, q+o 2*32*128*2 = 16384 B
    assert O.decode_step_bytes([1], 32, 8, 128, 1) == 4096 + 4 + 16384
    # page size 64: a 65-token context reads 2 entries
    assert O.decode_step_bytes([65], 32, 8, 128, 64) == 65 * 4096 + 8 + 16384
    # extend pairs: n new tokens on c cached tokens see n*c + n(n+1)/2 (query, key) pairs
    for c, n in ((0, 1), (5, 3), (2048, 1024)):
        assert O.extend_flops([c], [c + n], 2, 8) == 4 * 2 * 8 * (n * c + n * (n + 1) // 2)


ALL_PINS = [pin_sdpa_library, pin_softmax_library, pin_permutation_invariance, pin_padding_invariance,
            pin_prefix_sharing, pin_chunk_split, pin_closed_forms, pin_metadata_running_totals,
            pin_metadata_page_list, pin_store, pin_byte_model]
