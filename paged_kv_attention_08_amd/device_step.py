"""One layer's paged-KV step on the GPU for a batch described on the host.

`DeviceStep` uploads a batch description (the `workloads.Workload` fields:
lengths, table rows, page table, new-page rows, cached K/V rows, q / k / v of
the new tokens) into device buffers and runs the library's calls on it in the
order the pages give (metadata, store before attention, then attention).
Everything it computes goes through the C ABI; this module only moves data.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (BatchTensors, KVPoolTensors, MetadataBuffers, build_attn_metadata, build_attn_metadata_store,
               kv_store, paged_decode_attn, paged_extend_attn, plan_view, workspace_bytes)

BF16_NAN_BITS = 0x7FC0


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a bf16 device tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def i32(a, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


class DeviceStep:
    """All device buffers of one batch of one layer, plus the four calls."""

    def __init__(self, w, device="cuda", o_fill_nan: bool = True, upload_chunk_rows: int = 1 << 18,
                 pool: KVPoolTensors = None):
        """pool: an existing (zeroed) pool view to fill, e.g. one layer of a
        multi-layer cache; by default a fresh pool is allocated."""
        self.w = w
        self.device = device
        N, Hkv, d = w.num_pool_rows, w.num_kv_heads, w.head_dim
        if pool is None:
            self.k_pool = torch.zeros((N, Hkv, d), dtype=torch.bfloat16, device=device)
            self.v_pool = torch.zeros((N, Hkv, d), dtype=torch.bfloat16, device=device)
        else:
            assert tuple(pool.k.shape) == (N, Hkv, d) and pool.page_size == w.page_size
            self.k_pool, self.v_pool = pool.k, pool.v
        rows = w.cached_rows
        for s in range(0, rows.size, upload_chunk_rows):
            r = torch.from_numpy(rows[s:s + upload_chunk_rows]).to(device)
            self.k_pool[r] = bf16_tensor(w.k_cached[s:s + upload_chunk_rows], device)
            self.v_pool[r] = bf16_tensor(w.v_cached[s:s + upload_chunk_rows], device)
        poison = torch.arange(w.poison_rows.start, w.poison_rows.stop, device=device)
        nan = torch.full((len(w.poison_rows), Hkv, d), float("nan"), dtype=torch.bfloat16, device=device)
        self.k_pool[poison] = nan
        self.v_pool[poison] = nan
        self.pool = KVPoolTensors(self.k_pool, self.v_pool, w.page_size)
        self.page_table = i32(w.page_table, device)
        self.batch = BatchTensors(i32(w.table_idx, device), i32(w.cached_len, device), i32(w.device_len, device),
                                  w.num_decode, w.num_tokens)
        self.alloc_rows = i32(w.alloc_rows, device)
        self.q = bf16_tensor(w.q, device)
        self.k_new = bf16_tensor(w.k_new, device)
        self.v_new = bf16_tensor(w.v_new, device)
        self.o = torch.full_like(self.q, float("nan")) if o_fill_nan else torch.zeros_like(self.q)
        self.meta = MetadataBuffers.allocate(w.num_reqs, w.num_tokens, w.num_qo_heads, w.num_kv_heads, device)
        nbytes = workspace_bytes(w.num_reqs, w.num_qo_heads, w.head_dim)
        self.workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=device)

    # -- the four entry points, in the order the learning notes give (metadata,
    #    store before attention, then attention) -------------------------------
    def metadata(self, stream=None):
        w = self.w
        build_attn_metadata(self.batch, self.page_table, w.page_size, w.num_pool_rows, self.alloc_rows,
                            w.num_qo_heads, w.num_kv_heads, self.meta, stream)

    def store(self, stream=None):
        kv_store(self.pool, self.k_new, self.v_new, self.meta.out_loc[:self.w.num_tokens], self.meta.status, stream)

    def metadata_store(self, stream=None):
        """metadata and store in one call (build_attn_metadata_store)."""
        w = self.w
        build_attn_metadata_store(self.batch, self.page_table, self.pool, self.alloc_rows, w.num_qo_heads, self.meta,
                                  self.k_new, self.v_new, stream)

    def decode(self, stream=None):
        paged_decode_attn(self.pool, self.page_table, self.batch, self.meta, self.q, self.o, self.w.sm_scale,
                          self.workspace, stream)

    def extend(self, stream=None):
        paged_extend_attn(self.pool, self.page_table, self.batch, self.meta, self.q, self.o, self.w.sm_scale,
                          None, stream)

    def run(self, stream=None, fused_store: bool = False):
        if fused_store:
            self.metadata_store(stream)
        else:
            self.metadata(stream)
            self.store(stream)
        self.decode(stream)
        self.extend(stream)

    # -- readback ----------------------------------------------------------------
    def status(self) -> int:
        return int(self.meta.status.item())

    def output_f64(self, rows) -> np.ndarray:
        idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=self.device)
        return self.o[idx].float().cpu().numpy().astype(np.float64)

    def pool_rows_bits(self, rows):
        idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=self.device)
        k = self.k_pool[idx].view(torch.int16).cpu().numpy().view(np.uint16)
        v = self.v_pool[idx].view(torch.int16).cpu().numpy().view(np.uint16)
        return k, v

    def snapshot_pool(self):
        """Device copies of the whole K and V pools (bit patterns)."""
        return self.k_pool.view(torch.int16).clone(), self.v_pool.view(torch.int16).clone()

    def plan_host(self):
        """The plan written by the last metadata call, copied to the host, with
        the layout that locates its work lists (see pkv_plan_view_layout)."""
        w = self.w
        view = plan_view(w.num_reqs, w.num_tokens, w.num_qo_heads, w.num_kv_heads)
        return self.meta.plan.cpu().numpy(), view

    def free(self):
        for name in list(self.__dict__):
            if isinstance(getattr(self, name), torch.Tensor):
                setattr(self, name, None)
        self.pool = None
        self.meta = None
        torch.cuda.empty_cache()
