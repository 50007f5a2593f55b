"""ctypes view of libpagedkv.so: the structs and prototypes of include/pagedkv.h."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

# PAGEDKV_LIB selects another build of the same library (for example one built
# with different tile sizes); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("PAGEDKV_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARGUMENT = 1
PKV_ERR_UNSUPPORTED = 2
PKV_ERR_WORKSPACE = 3
PKV_ERR_HIP = 4
PKV_ERR_HOST_ALLOC = 5
PKV_ERR_SCRATCH = 6
PKV_STATIC_SCRATCH_BYTES = 17039360

PKV_STATUS_BAD_OUT_LOC = 0x01
PKV_STATUS_BAD_LENGTHS = 0x02
PKV_STATUS_BAD_TABLE_IDX = 0x04
PKV_STATUS_BAD_PAGE_ROW = 0x08
PKV_STATUS_BAD_DECODE = 0x10
PKV_STATUS_TOKEN_COUNT = 0x20
PKV_STATUS_BAD_ALLOC = 0x40
PKV_STATUS_BAD_POSITION = 0x80
PKV_STATUS_OUT_OF_PAGES = 0x100
PKV_STATUS_FREE_OVERFLOW = 0x200


class KVPool(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("num_rows", c_int64), ("row_stride", c_int64),
                ("page_size", c_int32), ("num_kv_heads", c_int32), ("head_dim", c_int32), ("reserved", c_int32)]


class PageTable(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("num_rows", c_int32), ("width", c_int32)]


class Batch(ctypes.Structure):
    _fields_ = [("num_reqs", c_int32), ("num_decode", c_int32), ("num_tokens", c_int64),
                ("table_idx", c_void_p), ("cached_len", c_void_p), ("device_len", c_void_p)]


class AttnMetadata(ctypes.Structure):
    _fields_ = [("out_loc", c_void_p), ("positions", c_void_p), ("qo_indptr", c_void_p),
                ("kv_indptr", c_void_p), ("last_indices", c_void_p), ("plan", c_void_p),
                ("plan_bytes", c_size_t), ("status", c_void_p)]


PKV_LAYOUT_LAYER_FIRST = 0
PKV_LAYOUT_PAGE_FIRST = 1
PKV_LAYOUT_ROW_INTERLEAVED = 2


class KVCache(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("num_rows", c_int64), ("num_layers", c_int32), ("layout", c_int32),
                ("page_size", c_int32), ("num_kv_heads", c_int32), ("head_dim", c_int32), ("reserved", c_int32)]


class QKNorm(ctypes.Structure):
    _fields_ = [("q_weight", c_void_p), ("k_weight", c_void_p), ("eps", c_float), ("reserved", c_int32)]


class FreeList(ctypes.Structure):
    _fields_ = [("rows", c_void_p), ("state", c_void_p), ("capacity", c_int32), ("page_size", c_int32),
                ("num_pool_rows", c_int64)]


class DecodeGraphDesc(ctypes.Structure):
    _fields_ = [("pool", KVPool), ("page_table", PageTable), ("max_reqs", c_int32), ("dummy_table_row", c_int32),
                ("num_qo_heads", c_int32), ("sm_scale", c_float), ("table_idx", c_void_p), ("cached_len", c_void_p),
                ("device_len", c_void_p), ("alloc_rows", c_void_p), ("q", c_void_p), ("o", c_void_p),
                ("k_new", c_void_p), ("v_new", c_void_p), ("meta", AttnMetadata), ("workspace", c_void_p),
                ("workspace_bytes", c_size_t), ("reserved", c_int32)]


class PlanView(ctypes.Structure):
    _fields_ = [("header_offset", c_int64), ("decode_tile_ptr_offset", c_int64), ("extend_tiles_offset", c_int64),
                ("total_bytes", c_int64), ("decode_runs", c_int32), ("decode_group_heads", c_int32),
                ("decode_tile_keys", c_int32), ("extend_tile_tokens", c_int32)]


# name -> (restype, argtypes); the exports of include/pagedkv.h
PROTOTYPES = {
    "pkv_plan_bytes": (c_size_t, [c_int32, c_int64, c_int32, c_int32]),
    "paged_attn_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "kv_store": (c_int, [POINTER(KVPool), c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
    "build_attn_metadata_store": (c_int, [POINTER(Batch), POINTER(PageTable), POINTER(KVPool), c_void_p, c_int64,
                                          c_int32, POINTER(AttnMetadata), c_void_p, c_void_p, c_void_p]),
    "build_attn_metadata": (c_int, [POINTER(Batch), POINTER(PageTable), c_int32, c_int64, c_void_p, c_int64,
                                    c_int32, c_int32, POINTER(AttnMetadata), c_void_p]),
    "paged_decode_attn": (c_int, [POINTER(KVPool), POINTER(PageTable), POINTER(Batch), POINTER(AttnMetadata),
                                  c_void_p, c_void_p, c_int32, c_float, c_void_p, c_size_t, c_void_p]),
    "paged_extend_attn": (c_int, [POINTER(KVPool), POINTER(PageTable), POINTER(Batch), POINTER(AttnMetadata),
                                  c_void_p, c_void_p, c_int32, c_float, c_void_p, c_size_t, c_void_p]),
    "paged_decode_attn_static": (c_int, [POINTER(KVPool), POINTER(PageTable), POINTER(Batch), POINTER(AttnMetadata),
                                         c_void_p, c_void_p, c_int32, c_float, c_void_p]),
    "pkv_kv_cache_layer": (c_int, [POINTER(KVCache), c_int32, POINTER(KVPool)]),
    "pkv_rope_cos_sin_cache": (c_int, [c_void_p, c_int32, c_int32, ctypes.c_double, c_void_p]),
    "kv_store_rope": (c_int, [POINTER(KVPool), c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                              c_void_p, c_int32, POINTER(QKNorm), c_void_p, c_void_p]),
    "pkv_free_list_reset": (c_int, [POINTER(FreeList), c_int32, c_void_p]),
    "pkv_alloc_pages": (c_int, [POINTER(FreeList), POINTER(Batch), c_void_p, c_int64, c_void_p, c_void_p]),
    "pkv_free_pages": (c_int, [POINTER(FreeList), c_void_p, c_int32, c_void_p, c_void_p]),
    "pkv_decode_graph_create": (c_int, [POINTER(DecodeGraphDesc), POINTER(c_int32), c_int32, POINTER(c_void_p),
                                        c_void_p]),
    "pkv_decode_graph_replay": (c_int, [c_void_p, c_int32, POINTER(c_int32), c_void_p]),
    "pkv_plan_view_layout": (c_int, [c_int32, c_int64, c_int32, c_int32, POINTER(PlanView)]),
    "pkv_decode_graph_destroy": (c_int, [c_void_p]),
    "pkv_error_string": (ctypes.c_char_p, [c_int]),
    "pkv_last_hip_error": (c_int, []),
    "pkv_version": (c_int, []),
}

_LIB = None


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_attention_08_amd.build` "
                               "(the paged-KV path has no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB
