"""GPU parity of the step on one layer of a multi-layer KV cache (deep dive
6.2: one buffer for all layers, layer-first, page-first or row-interleaved), through the C
ABI: each layer holds different values on the same pages; running every
layer's store and attention gives each layer the oracle's result for its own
values, and never touches another layer's rows."""
import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_attention_08_amd as pkv
from tests import parity_checks as P
from tests.gpu_harness import DeviceStep, bf16_tensor, log
from workloads import configs

pytestmark = pytest.mark.gpu
L = 3


def layer_workload(w, layer):
    """Same batch and pages; the layer's values are the base values with rows
    rolled (cached) and tokens reversed (new rows, q), so layers differ."""
    if layer == 0:
        return w
    return dataclasses.replace(w, k_cached=np.roll(w.k_cached, layer, axis=0), v_cached=np.roll(w.v_cached, -layer, axis=0),
                               k_new=np.roll(w.k_new, layer, axis=0), v_new=np.roll(w.v_new, layer, axis=0),
                               q=np.roll(w.q, layer, axis=0))


@pytest.mark.parametrize("layout", [pkv.KVCacheTensors.LAYER_FIRST, pkv.KVCacheTensors.PAGE_FIRST,
                                    pkv.KVCacheTensors.ROW_INTERLEAVED],
                         ids=["layer_first", "page_first", "row_interleaved"])
@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "one_call"])
@pytest.mark.parametrize("cfg", [2, 5])
def test_each_layer_matches_oracle(layout, cfg, fused):
    """fused: metadata and store through build_attn_metadata_store, whose store
    workgroups take the layer's row stride."""
    w = configs.small(cfg)
    log(f"multi-layer cache layout {layout} config {cfg} fused {fused}: {w.summary()}")
    cache = pkv.KVCacheTensors(L, w.num_pool_rows, w.num_kv_heads, w.head_dim, w.page_size, layout)
    steps = [DeviceStep(layer_workload(w, l), pool=cache.layer(l)) for l in range(L)]
    torch.cuda.synchronize()
    snap = lambda s: (s.k_pool.clone(), s.v_pool.clone())
    before = [snap(s) for s in steps]
    for l, ds in enumerate(steps):
        if fused:
            ds.metadata_store()
        else:
            ds.metadata()
            ds.store()
        if w.num_decode:
            ds.decode()
        if w.num_decode < w.num_reqs:
            ds.extend()
        torch.cuda.synchronize()
        assert ds.status() == 0
        for m, other in enumerate(steps):  # no other layer's rows changed
            if m != l:
                assert torch.equal(other.k_pool.view(torch.int16), before[m][0].view(torch.int16)), (l, m)
                assert torch.equal(other.v_pool.view(torch.int16), before[m][1].view(torch.int16)), (l, m)
        before[l] = snap(ds)
    for l, ds in enumerate(steps):
        wl = ds.w
        ref = P.oracle_for(wl)
        P.check_store(ds, ref, wl)
        stats = P.check_attention(ds, ref["out"], wl, f"layer {l}")
        log(f"layer {l}: max-abs {stats['max_abs']:.2e}")
    for s in steps:
        s.free()
