"""GPU test of paged_decode_attn_static, the decode variant that allocates
nothing (its split-K workspace is the library's static device scratch),
through the C ABI.

Two calls in a row share the GPU's scratch, the second on a smaller batch
(fewer requests, a smaller query-head group): each call's outputs must be
bit-identical to paged_decode_attn's on the same inputs (same kernels, same
plan, another workspace address) and within the attention bar of the fp64
oracle.  The first batch's long contexts split every request over many
decode runs, so the merge reads partial states from the scratch.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_08_amd as pkv
from paged_kv_attention_08_amd.device_step import DeviceStep
from tests import parity_checks as P
from tests.gpu_harness import log
from workloads import configs

pytestmark = pytest.mark.gpu


def _decode_tokens(w):
    """Output rows of the real decode requests (one new token each)."""
    starts = P.token_starts(w)
    return [int(starts[i]) for i in range(w.num_decode) if not w.is_padding[i]]


def _run(w, label):
    log(f"static-scratch decode {label}: {w.summary()}")
    ds = DeviceStep(w)
    ds.metadata()
    ds.store()
    ds.decode()
    torch.cuda.synchronize()
    want = ds.o.clone()
    ds.o.fill_(float("nan"))
    torch.cuda.synchronize()
    log("  paged_decode_attn_static")
    pkv.paged_decode_attn_static(ds.pool, ds.page_table, ds.batch, ds.meta, ds.q, ds.o, w.sm_scale)
    torch.cuda.synchronize()
    assert ds.status() == 0, f"device status {ds.status():#x}"
    rows = torch.as_tensor(_decode_tokens(w), device=ds.device)
    assert torch.equal(ds.o[rows].view(torch.int16), want[rows].view(torch.int16)), "differs from paged_decode_attn"
    ref = P.oracle_for(w, extend_tokens={})
    stats = P.check_attention(ds, {t: ref["out"][t] for t in _decode_tokens(w)}, w, label)
    log(f"  ok {stats}")
    ds.free()


def test_static_scratch_decode_two_calls_second_smaller():
    # 64 query / 8 KV heads, 3 requests of 1500-2600 keys: split over many runs, merged
    _run(configs.small(4), "long contexts, group 8")
    # then a smaller batch: 16 query / 8 KV heads, 4 requests of 64-256 keys
    _run(configs.small(1), "tiny batch, group 2")


def test_static_scratch_refuses_groups_beyond_it():
    w = configs.small(1)
    ds = DeviceStep(w)
    try:
        hq = w.num_kv_heads * 9  # 9 query heads per KV head
        q = torch.zeros((w.num_tokens, hq, w.head_dim), dtype=torch.bfloat16, device=ds.device)
        meta = pkv.MetadataBuffers.allocate(w.num_reqs, w.num_tokens, hq, w.num_kv_heads, ds.device)
        with pytest.raises(pkv.PagedKVError) as e:
            pkv.paged_decode_attn_static(ds.pool, ds.page_table, ds.batch, meta, q, q.clone(), w.sm_scale)
        assert e.value.code == 6
    finally:
        ds.free()
