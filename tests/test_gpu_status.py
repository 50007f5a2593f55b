"""GPU tests of the device-side checks: requests, page-table entries and
lengths that are invalid on the device are skipped and reported through the
status word, the calls finish normally, and the valid requests of the same
batch keep their oracle results.  (Every bad value here is one the kernels
check before using it as an address.)"""
import numpy as np
import pytest
import torch

import paged_kv_attention_08_amd as pkv
from tests import parity_checks as P
from tests.gpu_harness import DeviceStep, log
from workloads import configs

pytestmark = pytest.mark.gpu


def run(ds, w):
    ds.metadata()
    ds.store()
    if w.num_decode:
        ds.decode()
    if w.num_decode < w.num_reqs:
        ds.extend()
    torch.cuda.synchronize()
    return ds.status()


def test_bad_table_idx_and_page_entry_skip_only_their_requests():
    w = configs.small(2)
    real = [i for i in range(w.num_decode) if not w.is_padding[i]]
    bad_req = real[3]
    victim = next(i for i in real if w.cached_len[i] > 12 and i != bad_req)
    ref = P.oracle_for(w)
    ds = DeviceStep(w)
    R, N = w.page_table.shape[0], w.num_pool_rows
    ds.batch.table_idx[bad_req] = R + 5                      # outside the page table
    ds.page_table[int(w.table_idx[victim]), 10] = N + 100   # a cached key's row outside the pool
    log(f"bad table_idx on request {bad_req}, bad entry on request {victim}")
    st = run(ds, w)
    assert st == (pkv.PKV_STATUS_BAD_TABLE_IDX | pkv.PKV_STATUS_BAD_PAGE_ROW), hex(st)
    assert int(ds.meta.out_loc[bad_req]) == -1 and int(ds.meta.positions[bad_req]) == -1
    assert torch.isnan(ds.o[bad_req].float()).all()         # skipped: never written
    assert torch.isfinite(ds.o[victim].float()).all()       # the bad key is masked, the rest attended
    keep = {i: ref["out"][i] for i in real if i not in (bad_req, victim)}
    P.check_attention(ds, keep, w, "valid requests next to bad ones")
    ds.free()


@pytest.mark.parametrize("case", ["cached_gt_device", "device_past_width", "decode_extend_len_2"])
def test_bad_lengths_are_reported(case):
    w = configs.small(5)
    ds = DeviceStep(w)
    W = w.page_table.shape[1]
    if case == "cached_gt_device":
        i = w.num_decode + 1
        ds.batch.cached_len[i] = int(w.device_len[i]) + 3
        want = pkv.PKV_STATUS_BAD_LENGTHS
    elif case == "device_past_width":
        i = w.num_decode - 1
        ds.batch.device_len[i] = W + 5
        ds.batch.cached_len[i] = W + 4
        want = pkv.PKV_STATUS_BAD_LENGTHS
    else:
        i = 2
        ds.batch.device_len[i] = int(w.device_len[i]) + 1
        want = pkv.PKV_STATUS_BAD_DECODE
    log(f"{case} on request {i}")
    st = run(ds, w)
    assert st & want, hex(st)
    # every output row is either untouched (NaN) or finite: nothing was read out of place
    o = ds.o.float()
    assert bool((torch.isnan(o).all(dim=-1) | torch.isfinite(o).all(dim=-1)).all())
    ds.free()


def test_kv_store_skips_bad_rows():
    """out_loc outside the pool is skipped and reported; -1 (an unmapped token)
    is skipped silently; the other rows are stored."""
    N, hkv, d = 64, 8, 128
    k_pool = torch.zeros((N, hkv, d), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    pool = pkv.KVPoolTensors(k_pool, v_pool)
    k_new = torch.randn((4, hkv, d), device="cuda").to(torch.bfloat16)
    v_new = torch.randn((4, hkv, d), device="cuda").to(torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.kv_store(pool, k_new, v_new, torch.tensor([3, -1, 9, 5], dtype=torch.int32, device="cuda"), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    pkv.kv_store(pool, k_new, v_new, torch.tensor([3, N, -2, 5], dtype=torch.int32, device="cuda"), status)
    torch.cuda.synchronize()
    assert int(status.item()) == pkv.PKV_STATUS_BAD_OUT_LOC
    for t, r in ((0, 3), (2, 9), (3, 5)):
        assert torch.equal(k_pool[r], k_new[t]) and torch.equal(v_pool[r], v_new[t])
    touched = {3, 5, 9}
    assert not any(k_pool[r].any() for r in range(N) if r not in touched)
