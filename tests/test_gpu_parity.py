"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small variants of the five workloads are checked on every output; the
full-size workloads (the sizes the benchmark times, in the same launch
configuration) are checked bit-exactly on metadata and store and on sampled
attention outputs.  Planted-spike cases pin the gather at specific positions
(first row, last row, split and page boundaries), where a dropped or shifted
key would otherwise hide in the small N(0,1) outputs of long contexts.
"""
import numpy as np
import pytest
import torch

from workloads import RequestSpec, build_workload, configs
from tests.gpu_harness import DeviceStep, log
from tests import parity_checks as P

pytestmark = pytest.mark.gpu


def run_case(w, decode_requests=None, extend_tokens=None, label=""):
    log(f"case {label}: {w.summary()}")
    ds = DeviceStep(w)
    log("  device step")
    ds.run()
    torch.cuda.synchronize()
    log("  device step done")
    assert ds.status() == 0, f"device status bits {ds.status():#x}"
    ref = P.oracle_for(w, decode_requests, extend_tokens)
    P.check_metadata(ds, ref, w)
    P.check_store(ds, ref, w)
    P.real_outputs_finite(ds, w)
    stats = P.check_attention(ds, ref["out"], w, label)
    log(f"  ok {stats}")
    return ds, ref, stats


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_small_config(cfg):
    w = configs.small(cfg)
    ds, _, _ = run_case(w, label=f"small{cfg}")
    ds.free()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_config(cfg):
    w = configs.FULL[cfg]()
    dec = None
    if w.num_decode > 64:
        rng = np.random.default_rng(cfg)
        dec = sorted(set(rng.choice(w.num_decode, 48, replace=False).tolist()) | {0, w.num_decode - 1})
    elif cfg == 4:
        dec = [0, 7, 15, 31]
    ext = P.sample_tokens(w, per_request=6, seed=cfg) if w.num_decode < w.num_reqs else None
    ds, _, _ = run_case(w, decode_requests=dec, extend_tokens=ext, label=f"full{cfg}")
    ds.free()


def _plant(w, positions):
    """Make key `positions[i]` of request i dominate every query of the
    request and give it a one-hot V; returns the expected one-hot rows."""
    d = w.head_dim
    row_of_cached = {int(r): n for n, r in enumerate(w.cached_rows)}
    starts = P.token_starts(w)
    expect = {}
    rng = np.random.default_rng(17)
    for i, j in positions.items():
        t0, t1 = starts[i], starts[i + 1]
        c = int(w.cached_len[i])
        u = rng.normal(size=d).astype(np.float32)
        ub = (np.frombuffer(u.tobytes(), dtype=np.uint32) + 0x7FFF + ((np.frombuffer(u.tobytes(), dtype=np.uint32) >> 16) & 1)) >> 16
        ub = ub.astype(np.uint16)
        w.q[t0:t1, :, :] = ub[None, None, :]
        kb = (np.frombuffer((u * 4).astype(np.float32).tobytes(), dtype=np.uint32))
        kb = ((kb + 0x7FFF + ((kb >> 16) & 1)) >> 16).astype(np.uint16)
        onehot = np.zeros(d, dtype=np.uint16)
        hot = (i * 7) % d
        onehot[hot] = 0x3F80  # 1.0
        if j < c:
            n = row_of_cached[int(w.page_table[w.table_idx[i], j])]
            w.k_cached[n, :, :] = kb[None, :]
            w.v_cached[n, :, :] = onehot[None, :]
        else:
            t = t0 + (j - c)
            w.k_new[t, :, :] = kb[None, :]
            w.v_new[t, :, :] = onehot[None, :]
        vec = np.zeros(d)
        vec[hot] = 1.0
        expect[i] = (vec, j)
    return expect


@pytest.mark.parametrize("kind", ["decode", "extend", "page64"])
def test_planted_spikes(kind):
    if kind == "decode":
        w = configs.serving_decode(seed=31, real=12, padded_to=16, lo=1500, hi=2600, num_pool_rows=1 << 16)
        pos = [0, 1, 31, 32, 63, 64, 255, 256, 511, 512, 1023, None]
    elif kind == "extend":
        w = configs.extend_radix(seed=32, nreq=3, prefix=256, tail_hi=200, chunk=300, num_pool_rows=1 << 14)
        pos = [0, 270, None]
    else:
        w = configs.mixed_page64(seed=33, ndec=8, dec_lo=600, dec_hi=900, next_=2, pre_hi=300, new_tokens=130,
                                 num_pool_rows=64 * 128)
        pos = [0, 63, 64, 127, 128, 511, 512, None, 64, 0]
    positions = {}
    real = [i for i in range(w.num_reqs) if not w.is_padding[i]]
    for n, i in enumerate(real):
        p = pos[n % len(pos)]
        dl = int(w.device_len[i])
        positions[i] = dl - 1 if p is None or p >= dl else p
    expect = _plant(w, positions)
    ds, ref, _ = run_case(w, label=f"spike-{kind}")
    starts = P.token_starts(w)
    for i, (vec, j) in expect.items():
        c = int(w.cached_len[i])
        for t in range(starts[i], starts[i + 1]):
            if c + (t - starts[i]) < j:
                continue  # the planted key is not visible to this token
            got = ds.output_f64([t])[0]
            err = np.abs(got - vec[None, :]).max()
            assert err < 2e-2, f"request {i} token {t} planted key {j}: max err {err:.3e}"
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


def _edge_workloads():
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
    # one-workgroup plan kernel (512 new tokens) and launches a kernel for them
    for nreq in (512, 513):
        lens = [(37 * k) % 300 + 1 for k in range(nreq)]
        reqs = [RequestSpec(l, l + 1) for l in lens]
        cases.append((f"meta{nreq}", build_workload(f"meta{nreq}", 62 + nreq % 2, reqs, num_qo_heads=32,
                                                    num_kv_heads=8, head_dim=128, page_size=1,
                                                    num_pool_rows=1 << 18, num_decode=nreq)))
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
