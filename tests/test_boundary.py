"""CPU tests of the C ABI boundary: the library loads, exports every function
include/pagedkv.h declares, and rejects bad host-side arguments before any
launch (no GPU is touched: every call here returns during host validation)."""
import ctypes
import os
import re

import pytest

from paged_kv_attention_08_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("kv_store", "build_attn_metadata", "paged_decode_attn", "paged_extend_attn"):
        assert n in names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libpagedkv.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def test_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in pagedkv.h but not exported"
        assert n in _lib.PROTOTYPES, f"{n} has no ctypes prototype"


def test_version_and_strings(lib):
    assert lib.pkv_version() == 2
    for code in range(7):
        assert lib.pkv_error_string(code)
    assert lib.pkv_last_hip_error() == 0


def test_size_queries(lib):
    assert lib.pkv_plan_bytes(256, 256, 32, 8) > 0
    assert lib.pkv_plan_bytes(0, 0, 32, 8) > 0
    assert lib.pkv_plan_bytes(256, 256, 32, 7) == 0      # Hq % Hkv != 0
    assert lib.pkv_plan_bytes(256, 256, 64, 2) == 0      # group 32 > 16
    assert lib.pkv_plan_bytes(-1, 0, 32, 8) == 0
    assert lib.pkv_plan_bytes(10, 100, 32, 8) <= lib.pkv_plan_bytes(20, 100, 32, 8)


def test_plan_view_layout(lib):
    """The plan's documented work-list offsets fit inside pkv_plan_bytes and do
    not overlap, for a few batch shapes; bad head counts are rejected."""
    for (B, T, hq, hkv) in [(256, 256, 32, 8), (68, 8256, 32, 8), (32, 32, 64, 8), (3, 40, 12, 3), (0, 0, 8, 8)]:
        v = _lib.PlanView()
        assert lib.pkv_plan_view_layout(B, T, hq, hkv, ctypes.byref(v)) == _lib.PKV_OK
        assert v.total_bytes == lib.pkv_plan_bytes(B, T, hq, hkv)
        assert v.header_offset == 0 and v.decode_tile_ptr_offset >= 32
        assert v.extend_tiles_offset >= v.decode_tile_ptr_offset + 4 * (B + 1)
        tiles_cap = -(-T // v.extend_tile_tokens) + B
        assert v.extend_tiles_offset + 8 * tiles_cap <= v.total_bytes
        assert v.decode_tile_keys == 32 and v.extend_tile_tokens == 256 // (hq // hkv)
        assert v.decode_group_heads in (1, 2, 4, 8) and hkv % v.decode_group_heads == 0
        assert v.decode_runs * v.decode_group_heads == 2048
    v = _lib.PlanView()
    assert lib.pkv_plan_view_layout(8, 8, 32, 7, ctypes.byref(v)) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_plan_view_layout(8, 8, 64, 2, ctypes.byref(v)) == _lib.PKV_ERR_UNSUPPORTED
    assert lib.pkv_plan_view_layout(-1, 8, 32, 8, ctypes.byref(v)) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_plan_view_layout(8, 8, 32, 8, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.paged_attn_workspace_bytes(256, 32, 128) > 0
    assert lib.paged_attn_workspace_bytes(256, 32, 64) == 0
    assert lib.paged_attn_workspace_bytes(256, 0, 128) == 0


FAKE = 0x1000  # never dereferenced: every call below fails host validation first


def pool(**kw):
    p = dict(k=FAKE, v=FAKE, num_rows=4096, row_stride=1024, page_size=1, num_kv_heads=8, head_dim=128, reserved=0)
    p.update(kw)
    return _lib.KVPool(**p)


def batch(**kw):
    b = dict(num_reqs=4, num_decode=4, num_tokens=4, table_idx=FAKE, cached_len=FAKE, device_len=FAKE)
    b.update(kw)
    return _lib.Batch(**b)


def table(**kw):
    t = dict(data=FAKE, num_rows=5, width=288)
    t.update(kw)
    return _lib.PageTable(**t)


def meta(**kw):
    m = dict(out_loc=FAKE, positions=FAKE, qo_indptr=FAKE, kv_indptr=FAKE, last_indices=FAKE, plan=FAKE,
             plan_bytes=1 << 20, status=None)
    m.update(kw)
    return _lib.AttnMetadata(**m)


B = ctypes.byref


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(head_dim=64), _lib.PKV_ERR_UNSUPPORTED),
    (dict(page_size=3), _lib.PKV_ERR_UNSUPPORTED),
    (dict(page_size=128, num_rows=4096), _lib.PKV_ERR_UNSUPPORTED),
    (dict(num_rows=4095, page_size=2), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(num_rows=1 << 31), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(row_stride=1000), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(row_stride=1028), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(row_stride=1 << 31), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(reserved=1), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(k=FAKE + 2), _lib.PKV_ERR_INVALID_ARGUMENT),
])
def test_kv_store_rejects_bad_pool(lib, kw, code):
    assert lib.kv_store(B(pool(**kw)), FAKE, FAKE, FAKE, 4, None, None) == code


def test_kv_store_rejects_bad_buffers(lib):
    assert lib.kv_store(None, FAKE, FAKE, FAKE, 4, None, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.kv_store(B(pool()), None, FAKE, FAKE, 4, None, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.kv_store(B(pool()), FAKE, FAKE, None, 4, None, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.kv_store(B(pool()), FAKE, FAKE, FAKE, -1, None, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    # zero tokens is a no-op that launches nothing
    assert lib.kv_store(B(pool()), None, None, None, 0, None, None) == _lib.PKV_OK


def _meta_call(lib, b=None, t=None, s=1, rows=4096, alloc=FAKE, nalloc=4, hq=32, hkv=8, m=None):
    return lib.build_attn_metadata(B(b or batch()), B(t or table()), s, rows, alloc, nalloc, hq, hkv, B(m or meta()),
                                   None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=batch(num_reqs=-1)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(b=batch(num_decode=5)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(b=batch(table_idx=None)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(b=batch(num_tokens=1 << 31)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(t=table(width=100)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(t=table(data=None)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(s=48), _lib.PKV_ERR_UNSUPPORTED),
    (dict(rows=4097, s=2), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(alloc=None), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(nalloc=-2), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(hq=30), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(hq=32, hkv=1), _lib.PKV_ERR_UNSUPPORTED),
    (dict(m=meta(plan_bytes=16)), _lib.PKV_ERR_WORKSPACE),
    (dict(m=meta(plan=None)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(m=meta(out_loc=None)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(m=meta(plan=FAKE + 4)), _lib.PKV_ERR_INVALID_ARGUMENT),
])
def test_build_attn_metadata_rejects(lib, kw, code):
    assert _meta_call(lib, **kw) == code


@pytest.mark.parametrize("fn", ["paged_decode_attn", "paged_extend_attn"])
@pytest.mark.parametrize("kw,code", [
    (dict(p=pool(head_dim=256)), _lib.PKV_ERR_UNSUPPORTED),
    (dict(hq=12), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(hq=8 * 17), _lib.PKV_ERR_UNSUPPORTED),
    (dict(scale=0.0), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(q=None), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(m=meta(plan_bytes=8)), _lib.PKV_ERR_WORKSPACE),
    (dict(t=table(width=31)), _lib.PKV_ERR_INVALID_ARGUMENT),
])
def test_attention_rejects(lib, fn, kw, code):
    f = getattr(lib, fn)
    p = kw.get("p", pool())
    t = kw.get("t", table())
    m = kw.get("m", meta())
    assert f(B(p), B(t), B(batch()), B(m), kw.get("q", FAKE), FAKE, kw.get("hq", 32), kw.get("scale", 0.088),
             FAKE, 1 << 30, None) == code


def test_decode_rejects_small_workspace(lib):
    need = lib.paged_attn_workspace_bytes(4, 32, 128)
    assert lib.paged_decode_attn(B(pool()), B(table()), B(batch()), B(meta()), FAKE, FAKE, 32, 0.088, FAKE,
                                 need - 16, None) == _lib.PKV_ERR_WORKSPACE
    assert lib.paged_decode_attn(B(pool()), B(table()), B(batch()), B(meta()), FAKE, FAKE, 32, 0.088, None,
                                 need, None) == _lib.PKV_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw,code", [
    (dict(p=pool(head_dim=256)), _lib.PKV_ERR_UNSUPPORTED),
    (dict(hq=12), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(hq=8 * 17), _lib.PKV_ERR_UNSUPPORTED),
    (dict(hq=8 * 9), _lib.PKV_ERR_SCRATCH),     # 9 query heads per KV head: beyond the static scratch
    (dict(hq=8 * 16), _lib.PKV_ERR_SCRATCH),
    (dict(scale=0.0), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(q=None), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(m=meta(plan_bytes=8)), _lib.PKV_ERR_WORKSPACE),
])
def test_static_decode_rejects(lib, kw, code):
    """The no-allocation decode variant checks like paged_decode_attn and
    refuses groups its static scratch cannot hold, all before touching a device."""
    p = kw.get("p", pool())
    m = kw.get("m", meta())
    assert lib.paged_decode_attn_static(B(p), B(table()), B(batch()), B(m), kw.get("q", FAKE), FAKE,
                                        kw.get("hq", 32), kw.get("scale", 0.088), None) == code


def test_static_scratch_size_is_the_stated_one(lib):
    # 2048 wavefronts x 2 pieces x 8 heads x (128 + 2) floats, the workspace of an 8-head group
    assert _lib.PKV_STATIC_SCRATCH_BYTES == 2048 * 2 * 8 * 130 * 4
    assert lib.paged_attn_workspace_bytes(1, 8, 128) == _lib.PKV_STATIC_SCRATCH_BYTES
    assert lib.paged_attn_workspace_bytes(1, 16, 128) > _lib.PKV_STATIC_SCRATCH_BYTES


def test_metadata_store_rejects(lib):
    """build_attn_metadata_store checks like its two calls, before any launch."""
    f = lib.build_attn_metadata_store
    ok = dict(b=batch(), t=table(), p=pool(), alloc=FAKE, n=4, hq=32, m=meta(), k=FAKE, v=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(B(a["b"]), B(a["t"]), B(a["p"]), a["alloc"], a["n"], a["hq"], B(a["m"]), a["k"], a["v"], None)

    assert call(p=pool(head_dim=64)) == _lib.PKV_ERR_UNSUPPORTED
    assert call(p=pool(k=None)) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert call(k=None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert call(v=FAKE + 4) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert call(hq=12) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert call(alloc=None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert call(m=meta(plan_bytes=8)) == _lib.PKV_ERR_WORKSPACE
    assert call(t=table(width=31)) == _lib.PKV_ERR_INVALID_ARGUMENT


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _lib.lib()


def _rope_call(lib, pool_kw=None, q=FAKE, hq=32, k=FAKE, v=FAKE, out_loc=FAKE, positions=FAKE, t=4, cache=FAKE,
               max_pos=4096, norm=None):
    p = pool(**(pool_kw or {}))
    return lib.kv_store_rope(ctypes.byref(p), q, hq, k, v, out_loc, positions, t, cache, max_pos,
                             ctypes.byref(norm) if norm is not None else None, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(pool_kw=dict(head_dim=64)), _lib.PKV_ERR_UNSUPPORTED),
    (dict(hq=0), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(hq=12), _lib.PKV_ERR_INVALID_ARGUMENT),       # not a multiple of Hkv = 8
    (dict(t=-1), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(cache=None), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(cache=FAKE + 4), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(max_pos=0), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(q=None), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 8), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(positions=None), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(out_loc=None), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(norm=_lib.QKNorm(None, FAKE, 1e-6, 0)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(norm=_lib.QKNorm(FAKE, FAKE, -1.0, 0)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(norm=_lib.QKNorm(FAKE, FAKE, float("nan"), 0)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(norm=_lib.QKNorm(FAKE, FAKE, 1e-6, 1)), _lib.PKV_ERR_INVALID_ARGUMENT),
    (dict(t=0), _lib.PKV_OK),                             # nothing to do: returns before any launch
])
def test_kv_store_rope_rejects(lib, kw, code):
    assert _rope_call(lib, **kw) == code


@pytest.mark.parametrize("args,code", [
    ((None, 4096, 128, 1e4), _lib.PKV_ERR_INVALID_ARGUMENT),
    ((FAKE + 4, 4096, 128, 1e4), _lib.PKV_ERR_INVALID_ARGUMENT),
    ((FAKE, 0, 128, 1e4), _lib.PKV_ERR_INVALID_ARGUMENT),
    ((FAKE, 4096, 64, 1e4), _lib.PKV_ERR_UNSUPPORTED),
    ((FAKE, 4096, 128, 1.0), _lib.PKV_ERR_INVALID_ARGUMENT),
    ((FAKE, 4096, 128, float("inf")), _lib.PKV_ERR_INVALID_ARGUMENT),
])
def test_rope_cache_rejects(lib, args, code):
    assert lib.pkv_rope_cos_sin_cache(*args, None) == code


def test_decode_graph_rejects_before_capture(lib):
    d = _lib.DecodeGraphDesc()
    sizes = (ctypes.c_int32 * 3)(1, 2, 4)
    h = ctypes.c_void_p()
    assert lib.pkv_decode_graph_create(None, sizes, 3, ctypes.byref(h), FAKE) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_decode_graph_create(ctypes.byref(d), sizes, 3, ctypes.byref(h), FAKE) == \
        _lib.PKV_ERR_INVALID_ARGUMENT                     # max_reqs 0, null buffers
    d.max_reqs = 4
    for name in ("table_idx", "cached_len", "device_len", "alloc_rows", "q", "o", "k_new", "v_new"):
        setattr(d, name, FAKE)
    d.page_table = _lib.PageTable(FAKE, 8, 32)
    d.dummy_table_row = 8                                 # outside the table
    assert lib.pkv_decode_graph_create(ctypes.byref(d), sizes, 3, ctypes.byref(h), FAKE) == \
        _lib.PKV_ERR_INVALID_ARGUMENT
    d.dummy_table_row = 7
    bad = (ctypes.c_int32 * 3)(1, 4, 2)                   # not increasing
    assert lib.pkv_decode_graph_create(ctypes.byref(d), bad, 3, ctypes.byref(h), FAKE) == _lib.PKV_ERR_INVALID_ARGUMENT
    big = (ctypes.c_int32 * 3)(1, 2, 8)                   # beyond max_reqs
    assert lib.pkv_decode_graph_create(ctypes.byref(d), big, 3, ctypes.byref(h), FAKE) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_decode_graph_create(ctypes.byref(d), sizes, 3, ctypes.byref(h), None) == \
        _lib.PKV_ERR_INVALID_ARGUMENT                     # the default stream cannot be captured
    assert lib.pkv_decode_graph_replay(None, 1, None, FAKE) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_decode_graph_destroy(None) == _lib.PKV_ERR_INVALID_ARGUMENT


def test_page_allocator_rejects(lib):
    fl = _lib.FreeList(FAKE, FAKE, 64, 16, 4096)
    b = batch()
    assert lib.pkv_alloc_pages(None, B(b), FAKE, 8, None, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_alloc_pages(B(_lib.FreeList(FAKE, FAKE, 64, 3, 4096)), B(b), FAKE, 8, None, None) == \
        _lib.PKV_ERR_UNSUPPORTED
    assert lib.pkv_alloc_pages(B(_lib.FreeList(FAKE, FAKE, 0, 16, 4096)), B(b), FAKE, 8, None, None) == \
        _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_alloc_pages(B(_lib.FreeList(FAKE, FAKE, 64, 16, 4095)), B(b), FAKE, 8, None, None) == \
        _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_alloc_pages(B(fl), B(b), None, 8, None, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_alloc_pages(B(fl), B(b), FAKE, -1, None, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_alloc_pages(B(fl), B(batch(num_reqs=0, num_decode=0, num_tokens=0)), None, 0, None, None) == \
        _lib.PKV_OK                                        # empty batch: nothing launched
    assert lib.pkv_free_pages(B(fl), None, 4, None, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_free_pages(B(fl), FAKE, -1, None, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_free_pages(B(fl), None, 0, None, None) == _lib.PKV_OK
    assert lib.pkv_free_list_reset(B(fl), 65, None) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_free_list_reset(B(fl), -1, None) == _lib.PKV_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("layout", [_lib.PKV_LAYOUT_LAYER_FIRST, _lib.PKV_LAYOUT_PAGE_FIRST,
                                    _lib.PKV_LAYOUT_ROW_INTERLEAVED])
def test_kv_cache_layer_pointers(lib, layout):
    """Host-only pointer arithmetic of the multi-layer cache (nothing launched)."""
    base, L, N, hkv, d = 1 << 20, 3, 4096, 8, 128
    row = hkv * d
    c = _lib.KVCache(base, N, L, layout, 16, hkv, d, 0)
    for layer in range(L):
        p = _lib.KVPool()
        assert lib.pkv_kv_cache_layer(B(c), layer, B(p)) == _lib.PKV_OK
        if layout == _lib.PKV_LAYOUT_LAYER_FIRST:
            k_elem, v_elem, stride = layer * N * row, (L + layer) * N * row, row
        elif layout == _lib.PKV_LAYOUT_PAGE_FIRST:
            k_elem, v_elem, stride = layer * row, N * L * row + layer * row, L * row
        else:
            k_elem, v_elem, stride = 2 * layer * row, 2 * layer * row + row, 2 * L * row
        assert (p.k, p.v, p.row_stride) == (base + 2 * k_elem, base + 2 * v_elem, stride)
        assert (p.num_rows, p.page_size, p.num_kv_heads, p.head_dim) == (N, 16, hkv, d)
    p = _lib.KVPool()
    assert lib.pkv_kv_cache_layer(B(c), L, B(p)) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_kv_cache_layer(B(c), -1, B(p)) == _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_kv_cache_layer(B(_lib.KVCache(base, N, L, 3, 16, hkv, d, 0)), 0, B(p)) == \
        _lib.PKV_ERR_INVALID_ARGUMENT
    assert lib.pkv_kv_cache_layer(B(_lib.KVCache(base, N, L, layout, 16, hkv, 64, 0)), 0, B(p)) == \
        _lib.PKV_ERR_UNSUPPORTED
    assert lib.pkv_kv_cache_layer(B(_lib.KVCache(base, N, L, layout, 3, hkv, d, 0)), 0, B(p)) == \
        _lib.PKV_ERR_UNSUPPORTED
    assert lib.pkv_kv_cache_layer(B(_lib.KVCache(base + 8, N, L, layout, 16, hkv, d, 0)), 0, B(p)) == \
        _lib.PKV_ERR_INVALID_ARGUMENT
