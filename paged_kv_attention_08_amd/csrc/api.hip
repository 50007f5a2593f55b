// extern "C" entry points: host-side argument checks, then launches on the
// caller's stream.  Nothing here allocates, frees or synchronises.
#include <cmath>
#include <mutex>

#include "kernels.hpp"

using namespace pkv;

// Workspace of paged_decode_attn_static: the split-K partial states of up to
// 8 query heads per KV head, one copy per GPU for the life of the process.  In
// host code its name is a host-side stand-in, not a device address: only the
// per-device address that hipGetSymbolAddress returns is passed to kernels.
static_assert(decode_ws_floats(8) * 4 == PKV_STATIC_SCRATCH_BYTES, "header states the scratch size");
static __device__ __align__(256) float scratch[PKV_STATIC_SCRATCH_BYTES / 4];

namespace pkv {

thread_local int g_last_hip_error = 0;

int hip_failed(hipError_t e) {
  g_last_hip_error = (int)e;
  return PKV_ERR_HIP;
}

}  // namespace pkv

namespace {


bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_le64(int32_t s) { return s >= 1 && s <= 64 && (s & (s - 1)) == 0; }

int log2i(int32_t s) {
  int k = 0;
  while ((1 << k) < s) ++k;
  return k;
}

int check_heads(int32_t hq, int32_t hkv) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return PKV_ERR_INVALID_ARGUMENT;
  if (hq / hkv > kMaxGroup) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

int check_pool(const pkv_kv_pool* p) {
  if (!p || !p->k || !p->v) return PKV_ERR_INVALID_ARGUMENT;
  if (p->head_dim != kHeadDim) return PKV_ERR_UNSUPPORTED;
  if (!pow2_le64(p->page_size)) return PKV_ERR_UNSUPPORTED;
  if (p->num_kv_heads <= 0 || p->reserved != 0) return PKV_ERR_INVALID_ARGUMENT;
  if (p->num_rows <= 0 || p->num_rows >= (int64_t(1) << 31) || p->num_rows % p->page_size != 0)
    return PKV_ERR_INVALID_ARGUMENT;
  if (p->row_stride < (int64_t)p->num_kv_heads * p->head_dim || p->row_stride % 8 != 0 ||
      p->row_stride >= (int64_t(1) << 31))
    return PKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(p->k) || !aligned16(p->v)) return PKV_ERR_INVALID_ARGUMENT;
  return PKV_OK;
}

int check_batch(const pkv_batch* b) {
  if (!b) return PKV_ERR_INVALID_ARGUMENT;
  if (b->num_reqs < 0 || b->num_decode < 0 || b->num_decode > b->num_reqs) return PKV_ERR_INVALID_ARGUMENT;
  if (b->num_tokens < 0 || b->num_tokens >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARGUMENT;
  if (b->num_reqs > 0 && (!b->table_idx || !b->cached_len || !b->device_len)) return PKV_ERR_INVALID_ARGUMENT;
  return PKV_OK;
}

int check_page_table(const pkv_page_table* t) {
  if (!t || !t->data || t->num_rows <= 0 || t->width <= 0 || t->width % 32 != 0) return PKV_ERR_INVALID_ARGUMENT;
  return PKV_OK;
}

int check_meta_common(const pkv_attn_metadata* m, const pkv_batch* b, int32_t group, int32_t hkv, PlanLayout* L) {
  if (!m || !m->qo_indptr || !m->kv_indptr || !m->plan) return PKV_ERR_INVALID_ARGUMENT;
  if (b->num_reqs > 0 && !m->last_indices) return PKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(m->plan)) return PKV_ERR_INVALID_ARGUMENT;
  *L = plan_layout(b->num_reqs, b->num_tokens, group, hkv);
  if (m->plan_bytes < (size_t)L->total) return PKV_ERR_WORKSPACE;
  return PKV_OK;
}

int fill_attn_args(const pkv_kv_pool* pool, const pkv_page_table* pt, const pkv_batch* batch,
                   const pkv_attn_metadata* meta, const void* q, void* o, int32_t hq, float sm_scale,
                   AttnArgs* a) {
  int rc;
  if ((rc = check_pool(pool)) != PKV_OK) return rc;
  if ((rc = check_page_table(pt)) != PKV_OK) return rc;
  if ((rc = check_batch(batch)) != PKV_OK) return rc;
  if ((rc = check_heads(hq, pool->num_kv_heads)) != PKV_OK) return rc;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return PKV_ERR_INVALID_ARGUMENT;
  if (batch->num_tokens > 0 && (!q || !o || !aligned16(q) || !aligned16(o))) return PKV_ERR_INVALID_ARGUMENT;
  PlanLayout L;
  if ((rc = check_meta_common(meta, batch, hq / pool->num_kv_heads, pool->num_kv_heads, &L)) != PKV_OK) return rc;
  a->k_pool = static_cast<const uint16_t*>(pool->k);
  a->v_pool = static_cast<const uint16_t*>(pool->v);
  a->row_stride = pool->row_stride;
  a->num_pool_rows = pool->num_rows;
  a->page_table = pt->data;
  a->R = pt->num_rows;
  a->W = pt->width;
  a->B = batch->num_reqs;
  a->num_decode = batch->num_decode;
  a->T = batch->num_tokens;
  a->Hq = hq;
  a->Hkv = pool->num_kv_heads;
  a->group = hq / pool->num_kv_heads;
  a->scale_log2 = sm_scale * 1.4426950408889634f;
  a->table_idx = batch->table_idx;
  a->cached_len = batch->cached_len;
  a->device_len = batch->device_len;
  a->qo_indptr = meta->qo_indptr;
  a->q = static_cast<const uint16_t*>(q);
  a->o = static_cast<uint16_t*>(o);
  a->plan = static_cast<const char*>(meta->plan);
  a->layout = L;
  a->ws_acc = nullptr;
  a->ws_ml = nullptr;
  a->status = meta->status;
  return PKV_OK;
}

// The decode kernel's partial states; G = Hq / Hkv is at most min(Hq, 16).
size_t decode_ws_bytes(int32_t hq) {
  const int32_t gmax = hq < kMaxGroup ? hq : kMaxGroup;
  return (size_t)(decode_ws_floats(gmax) * 4);
}

}  // namespace

namespace pkv {

int prepare_metadata(const pkv_batch* batch, const pkv_page_table* page_table, int32_t page_size,
                     int64_t num_pool_rows, const int32_t* alloc_rows, int64_t num_alloc, int32_t num_qo_heads,
                     int32_t num_kv_heads, const pkv_attn_metadata* meta, MetaArgs* out) {
  int rc;
  if ((rc = check_batch(batch)) != PKV_OK) return rc;
  if ((rc = check_page_table(page_table)) != PKV_OK) return rc;
  if (!pow2_le64(page_size)) return PKV_ERR_UNSUPPORTED;
  if (num_pool_rows <= 0 || num_pool_rows >= (int64_t(1) << 31) || num_pool_rows % page_size != 0)
    return PKV_ERR_INVALID_ARGUMENT;
  if (num_alloc < 0 || (num_alloc > 0 && !alloc_rows)) return PKV_ERR_INVALID_ARGUMENT;
  if ((rc = check_heads(num_qo_heads, num_kv_heads)) != PKV_OK) return rc;
  PlanLayout L;
  if ((rc = check_meta_common(meta, batch, num_qo_heads / num_kv_heads, num_kv_heads, &L)) != PKV_OK) return rc;
  if (batch->num_tokens > 0 && (!meta->out_loc || !meta->positions)) return PKV_ERR_INVALID_ARGUMENT;
  MetaArgs a{};
  a.B = batch->num_reqs;
  a.num_decode = batch->num_decode;
  a.R = page_table->num_rows;
  a.W = page_table->width;
  a.page_shift = log2i(page_size);
  a.group = num_qo_heads / num_kv_heads;
  a.Hkv = num_kv_heads;
  a.T = batch->num_tokens;
  a.num_pool_rows = num_pool_rows;
  a.num_alloc = num_alloc;
  a.table_idx = batch->table_idx;
  a.cached_len = batch->cached_len;
  a.device_len = batch->device_len;
  a.page_table = page_table->data;
  a.alloc_rows = alloc_rows;
  a.out_loc = meta->out_loc;
  a.positions = meta->positions;
  a.qo_indptr = meta->qo_indptr;
  a.kv_indptr = meta->kv_indptr;
  a.last_indices = meta->last_indices;
  a.status = meta->status;
  a.plan = static_cast<char*>(meta->plan);
  a.layout = L;
  a.pad_from = INT32_MAX;
  a.dummy_row = 0;
  a.pad_table_idx = a.pad_cached_len = a.pad_device_len = a.pad_alloc_rows = nullptr;
  a.k_new = a.v_new = nullptr;
  a.k_pool = a.v_pool = nullptr;
  a.store_stride_vec = 0;
  a.store_row_vec = 0;
  a.map_blocks = 0;
  *out = a;
  return PKV_OK;
}

int prepare_metadata_store(const pkv_batch* batch, const pkv_page_table* page_table, const pkv_kv_pool* pool,
                           const int32_t* alloc_rows, int64_t num_alloc, int32_t num_qo_heads,
                           const pkv_attn_metadata* meta, const void* k_new, const void* v_new, MetaArgs* a,
                           StoreArgs* st) {
  int rc = check_pool(pool);
  if (rc != PKV_OK) return rc;
  if ((rc = prepare_metadata(batch, page_table, pool->page_size, pool->num_rows, alloc_rows, num_alloc, num_qo_heads,
                             pool->num_kv_heads, meta, a)) != PKV_OK)
    return rc;
  if (batch->num_tokens > 0 && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)))
    return PKV_ERR_INVALID_ARGUMENT;
  a->k_new = static_cast<const uint4*>(k_new);
  a->v_new = static_cast<const uint4*>(v_new);
  a->k_pool = static_cast<uint4*>(pool->k);
  a->v_pool = static_cast<uint4*>(pool->v);
  a->store_stride_vec = pool->row_stride / 8;
  a->store_row_vec = pool->num_kv_heads * pool->head_dim / 8;
  st->k_new = a->k_new;
  st->v_new = a->v_new;
  st->out_loc = meta->out_loc;
  st->k_pool = a->k_pool;
  st->v_pool = a->v_pool;
  st->num_tokens = batch->num_tokens;
  st->row_stride_vec = a->store_stride_vec;
  st->num_rows = pool->num_rows;
  st->row_vec = a->store_row_vec;
  st->status = meta->status;
  return PKV_OK;
}

hipError_t launch_metadata_store(const MetaArgs& a, const StoreArgs& st, hipStream_t s) {
  hipError_t e = launch_metadata(a, s);
  if (e != hipSuccess || st.num_tokens == 0 || metadata_stores_rows(a)) return e;
  return launch_kv_store(st, s);
}

}  // namespace pkv

extern "C" {

size_t pkv_plan_bytes(int32_t max_reqs, int64_t max_tokens, int32_t num_qo_heads, int32_t num_kv_heads) {
  if (max_reqs < 0 || max_tokens < 0 || check_heads(num_qo_heads, num_kv_heads) != PKV_OK) return 0;
  return (size_t)plan_layout(max_reqs, max_tokens, num_qo_heads / num_kv_heads, num_kv_heads).total;
}

size_t paged_attn_workspace_bytes(int32_t max_reqs, int32_t num_qo_heads, int32_t head_dim) {
  if (max_reqs < 0 || num_qo_heads <= 0 || head_dim != kHeadDim) return 0;
  return decode_ws_bytes(num_qo_heads);
}

int kv_store(const pkv_kv_pool* pool, const void* k_new, const void* v_new, const int32_t* out_loc,
             int64_t num_tokens, int32_t* status, void* stream) {
  int rc = check_pool(pool);
  if (rc != PKV_OK) return rc;
  if (num_tokens < 0) return PKV_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !out_loc || !aligned16(k_new) || !aligned16(v_new)) return PKV_ERR_INVALID_ARGUMENT;
  StoreArgs a;
  a.k_new = static_cast<const uint4*>(k_new);
  a.v_new = static_cast<const uint4*>(v_new);
  a.out_loc = out_loc;
  a.k_pool = static_cast<uint4*>(pool->k);
  a.v_pool = static_cast<uint4*>(pool->v);
  a.num_tokens = num_tokens;
  a.row_stride_vec = pool->row_stride / 8;
  a.num_rows = pool->num_rows;
  a.row_vec = pool->num_kv_heads * pool->head_dim / 8;
  a.status = status;
  hipError_t e = launch_kv_store(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

int build_attn_metadata(const pkv_batch* batch, const pkv_page_table* page_table, int32_t page_size,
                        int64_t num_pool_rows, const int32_t* alloc_rows, int64_t num_alloc,
                        int32_t num_qo_heads, int32_t num_kv_heads, const pkv_attn_metadata* meta,
                        void* stream) {
  MetaArgs a;
  const int rc = prepare_metadata(batch, page_table, page_size, num_pool_rows, alloc_rows, num_alloc, num_qo_heads,
                                  num_kv_heads, meta, &a);
  if (rc != PKV_OK) return rc;
  hipError_t e = launch_metadata(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

int build_attn_metadata_store(const pkv_batch* batch, const pkv_page_table* page_table, const pkv_kv_pool* pool,
                              const int32_t* alloc_rows, int64_t num_alloc, int32_t num_qo_heads,
                              const pkv_attn_metadata* meta, const void* k_new, const void* v_new, void* stream) {
  MetaArgs a;
  StoreArgs st;
  const int rc = prepare_metadata_store(batch, page_table, pool, alloc_rows, num_alloc, num_qo_heads, meta, k_new,
                                        v_new, &a, &st);
  if (rc != PKV_OK) return rc;
  hipError_t e = launch_metadata_store(a, st, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

int paged_decode_attn(const pkv_kv_pool* pool, const pkv_page_table* page_table, const pkv_batch* batch,
                      const pkv_attn_metadata* meta, const void* q, void* o, int32_t num_qo_heads,
                      float sm_scale, void* workspace, size_t workspace_bytes, void* stream) {
  AttnArgs a;
  int rc = fill_attn_args(pool, page_table, batch, meta, q, o, num_qo_heads, sm_scale, &a);
  if (rc != PKV_OK) return rc;
  if (batch->num_decode == 0) return PKV_OK;
  const size_t need = decode_ws_bytes(num_qo_heads);
  if (!workspace || !aligned16(workspace)) return PKV_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return PKV_ERR_WORKSPACE;
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = a.ws_acc + (int64_t)kDecodeWaves * 2 * a.group * kHeadDim;
  hipError_t e = launch_decode(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

int paged_extend_attn(const pkv_kv_pool* pool, const pkv_page_table* page_table, const pkv_batch* batch,
                      const pkv_attn_metadata* meta, const void* q, void* o, int32_t num_qo_heads,
                      float sm_scale, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  AttnArgs a;
  int rc = fill_attn_args(pool, page_table, batch, meta, q, o, num_qo_heads, sm_scale, &a);
  if (rc != PKV_OK) return rc;
  if (batch->num_decode >= batch->num_reqs) return PKV_OK;
  hipError_t e = launch_extend(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

// ---- the no-allocation decode variant: a static device array as workspace --

namespace {

constexpr int kScratchMaxGroup = 8;
constexpr int kScratchMaxDevices = 64;

std::mutex g_scratch_mutex;
float* g_scratch_ptr[kScratchMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t scratch_on_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

int paged_decode_attn_static(const pkv_kv_pool* pool, const pkv_page_table* page_table, const pkv_batch* batch,
                             const pkv_attn_metadata* meta, const void* q, void* o, int32_t num_qo_heads,
                             float sm_scale, void* stream) {
  AttnArgs a;
  int rc = fill_attn_args(pool, page_table, batch, meta, q, o, num_qo_heads, sm_scale, &a);
  if (rc != PKV_OK) return rc;
  if (a.group > kScratchMaxGroup) return PKV_ERR_SCRATCH;
  if (batch->num_decode == 0) return PKV_OK;
  float* ws = nullptr;
  hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return hip_failed(e);
  a.ws_acc = ws;
  a.ws_ml = ws + (int64_t)kDecodeWaves * 2 * a.group * kHeadDim;
  e = launch_decode(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

namespace {

int check_free_list(const pkv_free_list* f) {
  if (!f || !f->rows || !f->state || f->capacity <= 0) return PKV_ERR_INVALID_ARGUMENT;
  if (!pow2_le64(f->page_size)) return PKV_ERR_UNSUPPORTED;
  if (f->num_pool_rows <= 0 || f->num_pool_rows >= (int64_t(1) << 31) || f->num_pool_rows % f->page_size != 0)
    return PKV_ERR_INVALID_ARGUMENT;
  return PKV_OK;
}

AllocArgs alloc_args(const pkv_free_list* f, int32_t* status) {
  AllocArgs a{};
  a.rows = f->rows;
  a.state = f->state;
  a.capacity = f->capacity;
  a.page_size = f->page_size;
  a.num_pool_rows = f->num_pool_rows;
  a.status = status;
  return a;
}

}  // namespace

int pkv_free_list_reset(const pkv_free_list* free_list, int32_t num_free, void* stream) {
  int rc = check_free_list(free_list);
  if (rc != PKV_OK) return rc;
  if (num_free < 0 || num_free > free_list->capacity) return PKV_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_free_list_reset(free_list->state, num_free, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

int pkv_alloc_pages(const pkv_free_list* free_list, const pkv_batch* batch, int32_t* alloc_rows, int64_t max_alloc,
                    int32_t* status, void* stream) {
  int rc = check_free_list(free_list);
  if (rc != PKV_OK) return rc;
  if ((rc = check_batch(batch)) != PKV_OK) return rc;
  if (max_alloc < 0 || (max_alloc > 0 && !alloc_rows)) return PKV_ERR_INVALID_ARGUMENT;
  if (batch->num_reqs == 0) return PKV_OK;
  AllocArgs a = alloc_args(free_list, status);
  a.B = batch->num_reqs;
  a.cached_len = batch->cached_len;
  a.device_len = batch->device_len;
  a.alloc_rows = alloc_rows;
  a.max_alloc = max_alloc;
  hipError_t e = launch_alloc_pages(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

int pkv_free_pages(const pkv_free_list* free_list, const int32_t* rows, int32_t num_rows, int32_t* status,
                   void* stream) {
  int rc = check_free_list(free_list);
  if (rc != PKV_OK) return rc;
  if (num_rows < 0 || (num_rows > 0 && !rows)) return PKV_ERR_INVALID_ARGUMENT;
  if (num_rows == 0) return PKV_OK;
  AllocArgs a = alloc_args(free_list, status);
  a.free_rows = rows;
  a.num_free = num_rows;
  hipError_t e = launch_free_pages(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

int pkv_kv_cache_layer(const pkv_kv_cache* cache, int32_t layer_id, pkv_kv_pool* pool) {
  if (!cache || !pool || !cache->data || !aligned16(cache->data) || cache->reserved != 0) return PKV_ERR_INVALID_ARGUMENT;
  if (cache->num_layers <= 0 || layer_id < 0 || layer_id >= cache->num_layers) return PKV_ERR_INVALID_ARGUMENT;
  if (cache->layout != PKV_LAYOUT_LAYER_FIRST && cache->layout != PKV_LAYOUT_PAGE_FIRST &&
      cache->layout != PKV_LAYOUT_ROW_INTERLEAVED)
    return PKV_ERR_INVALID_ARGUMENT;
  if (cache->head_dim != kHeadDim) return PKV_ERR_UNSUPPORTED;
  if (cache->num_kv_heads <= 0 || cache->num_rows <= 0) return PKV_ERR_INVALID_ARGUMENT;
  const int64_t row = (int64_t)cache->num_kv_heads * cache->head_dim;  // elements of one layer's row
  const int64_t L = cache->num_layers, N = cache->num_rows;
  int64_t k_off, v_off, stride;
  if (cache->layout == PKV_LAYOUT_LAYER_FIRST) {
    k_off = (int64_t)layer_id * N * row;
    v_off = (L + layer_id) * N * row;
    stride = row;
  } else if (cache->layout == PKV_LAYOUT_PAGE_FIRST) {
    k_off = (int64_t)layer_id * row;
    v_off = N * L * row + (int64_t)layer_id * row;
    stride = L * row;
  } else {
    k_off = (int64_t)layer_id * 2 * row;
    v_off = k_off + row;
    stride = L * 2 * row;
  }
  pkv_kv_pool p;
  p.k = static_cast<uint16_t*>(cache->data) + k_off;
  p.v = static_cast<uint16_t*>(cache->data) + v_off;
  p.num_rows = N;
  p.row_stride = stride;
  p.page_size = cache->page_size;
  p.num_kv_heads = cache->num_kv_heads;
  p.head_dim = cache->head_dim;
  p.reserved = 0;
  const int rc = check_pool(&p);  // page size, row count and stride limits
  if (rc != PKV_OK) return rc;
  *pool = p;
  return PKV_OK;
}

int pkv_rope_cos_sin_cache(float* cache, int32_t max_position, int32_t head_dim, double base, void* stream) {
  if (!cache || !aligned16(cache) || max_position <= 0) return PKV_ERR_INVALID_ARGUMENT;
  if (head_dim != kHeadDim) return PKV_ERR_UNSUPPORTED;
  if (!(base > 1.0) || !std::isfinite(base)) return PKV_ERR_INVALID_ARGUMENT;
  RopeCacheArgs a;
  a.cache = cache;
  a.max_position = max_position;
  a.log2_base = std::log2(base);
  hipError_t e = launch_rope_cache(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

int kv_store_rope(const pkv_kv_pool* pool, void* q, int32_t num_qo_heads, const void* k_new, const void* v_new,
                  const int32_t* out_loc, const int32_t* positions, int64_t num_tokens,
                  const float* cos_sin_cache, int32_t max_position, const pkv_qk_norm* qk_norm,
                  int32_t* status, void* stream) {
  int rc = check_pool(pool);
  if (rc != PKV_OK) return rc;
  if (num_tokens < 0 || num_qo_heads <= 0 || num_qo_heads % pool->num_kv_heads != 0) return PKV_ERR_INVALID_ARGUMENT;
  if (max_position <= 0 || !cos_sin_cache || !aligned16(cos_sin_cache)) return PKV_ERR_INVALID_ARGUMENT;
  if (qk_norm && (!qk_norm->q_weight || !qk_norm->k_weight || !aligned16(qk_norm->q_weight) ||
                  !aligned16(qk_norm->k_weight) || !(qk_norm->eps >= 0.f) || qk_norm->reserved != 0))
    return PKV_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return PKV_OK;
  if (!q || !k_new || !v_new || !out_loc || !positions || !aligned16(q) || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_INVALID_ARGUMENT;
  RopeArgs a;
  a.q = static_cast<uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.out_loc = out_loc;
  a.positions = positions;
  a.cos_sin = cos_sin_cache;
  a.q_weight = qk_norm ? static_cast<const uint16_t*>(qk_norm->q_weight) : nullptr;
  a.k_weight = qk_norm ? static_cast<const uint16_t*>(qk_norm->k_weight) : nullptr;
  a.eps = qk_norm ? qk_norm->eps : 0.f;
  a.k_pool = static_cast<uint16_t*>(pool->k);
  a.v_pool = static_cast<uint16_t*>(pool->v);
  a.num_tokens = num_tokens;
  a.row_stride = pool->row_stride;
  a.num_rows = pool->num_rows;
  a.Hq = num_qo_heads;
  a.Hkv = pool->num_kv_heads;
  a.max_position = max_position;
  a.status = status;
  hipError_t e = launch_kv_store_rope(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_failed(e);
}

int pkv_plan_view_layout(int32_t max_reqs, int64_t max_tokens, int32_t num_qo_heads, int32_t num_kv_heads,
                         pkv_plan_view* view) {
  if (!view || max_reqs < 0 || max_tokens < 0) return PKV_ERR_INVALID_ARGUMENT;
  const int rc = check_heads(num_qo_heads, num_kv_heads);
  if (rc != PKV_OK) return rc;
  const PlanLayout L = plan_layout(max_reqs, max_tokens, num_qo_heads / num_kv_heads, num_kv_heads);
  const int32_t hg = decode_heads_per_group(num_kv_heads);
  view->header_offset = 0;
  view->decode_tile_ptr_offset = L.dec_tiles_off;
  view->extend_tiles_offset = L.tiles_off;
  view->total_bytes = L.total;
  view->decode_runs = kDecodeWaves / hg;
  view->decode_group_heads = hg;
  view->decode_tile_keys = kDecodeTileKeys;
  view->extend_tile_tokens = L.tile_q;
  return PKV_OK;
}

const char* pkv_error_string(int code) {
  switch (code) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "plan or workspace too small";
    case PKV_ERR_HIP: return "HIP launch failure";
    case PKV_ERR_HOST_ALLOC: return "host allocation failed";
    case PKV_ERR_SCRATCH: return "needs more than the static scratch holds";
    default: return "unknown error code";
  }
}

int pkv_last_hip_error(void) { return g_last_hip_error; }

int pkv_version(void) { return 2; }

}  // extern "C"
