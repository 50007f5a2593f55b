// Kernel argument blocks and launchers (internal to the library).
#pragma once

#include "common.hpp"

namespace pkv {

struct StoreArgs {
  const uint4* k_new;
  const uint4* v_new;
  const int32_t* out_loc;
  uint4* k_pool;
  uint4* v_pool;
  int64_t num_tokens;
  int64_t row_stride_vec;  // 16-byte vectors between pool rows
  int64_t num_rows;
  int32_t row_vec;         // 16-byte vectors per new row (Hkv * d * 2 / 16)
  int32_t* status;
};

struct RopeArgs {
  uint16_t* q;                // [T, Hq, 128], rotated in place
  const uint16_t* k_new;      // [T, Hkv, 128]
  const uint16_t* v_new;      // [T, Hkv, 128]
  const int32_t* out_loc;
  const int32_t* positions;
  const float* cos_sin;       // [max_position, 128]
  const uint16_t* q_weight;   // bf16 [128] or null (no norm)
  const uint16_t* k_weight;
  float eps;
  uint16_t* k_pool;
  uint16_t* v_pool;
  int64_t num_tokens;
  int64_t row_stride;         // elements between pool rows
  int64_t num_rows;
  int32_t Hq, Hkv, max_position;
  int32_t* status;
};

struct RopeCacheArgs {
  float* cache;
  int32_t max_position;
  double log2_base;
};

struct AllocArgs {
  int32_t* rows;              // ring of free page-start rows [capacity]
  int32_t* state;             // [2]: head, count
  int32_t capacity;
  int32_t page_size;
  int64_t num_pool_rows;
  // allocation
  int32_t B;
  const int32_t* cached_len;
  const int32_t* device_len;
  int32_t* alloc_rows;
  int64_t max_alloc;
  // freeing
  const int32_t* free_rows;
  int32_t num_free;
  int32_t* status;
};

struct MetaArgs {
  int32_t B, num_decode, R, W, page_shift, group, Hkv;
  int64_t T, num_pool_rows, num_alloc;
  const int32_t* table_idx;
  const int32_t* cached_len;
  const int32_t* device_len;
  int32_t* page_table;
  const int32_t* alloc_rows;
  int32_t* out_loc;
  int32_t* positions;
  int32_t* qo_indptr;
  int32_t* kv_indptr;
  int32_t* last_indices;
  int32_t* status;
  char* plan;
  PlanLayout layout;
  // Graph-replay padding: requests [pad_from, B) are dummy requests (table row
  // dummy_row, cached_len 0, device_len 1, their new row the dummy page's row 0)
  // whatever the batch arrays hold; plan_kernel writes those values (and the
  // dummy page's row 0 as their alloc entry) into the arrays below for the
  // later kernels.  pad_from = INT32_MAX: no padding.
  int32_t pad_from;
  int32_t dummy_row;
  int32_t* pad_table_idx;
  int32_t* pad_cached_len;
  int32_t* pad_device_len;
  int32_t* pad_alloc_rows;
  // Store in the metadata launch (build_attn_metadata_store): when k_new is
  // set, the map blocks of plan_kernel also copy the new K/V rows into the
  // pool.
  const uint4* k_new;
  const uint4* v_new;
  uint4* k_pool;
  uint4* v_pool;
  int64_t store_stride_vec;  // 16-byte vectors between pool rows
  int32_t store_row_vec;     // 16-byte vectors per K (or V) row of a token
  // workgroups 1..map_blocks of plan_kernel map the new tokens (0: a
  // token_kernel launch does); set by the launcher
  int32_t map_blocks;
};

struct AttnArgs {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int64_t row_stride;      // bf16 elements
  int64_t num_pool_rows;
  const int32_t* page_table;
  int32_t R, W;
  int32_t B, num_decode;
  int64_t T;
  int32_t Hq, Hkv, group;
  float scale_log2;        // sm_scale * log2(e)
  const int32_t* table_idx;
  const int32_t* cached_len;
  const int32_t* device_len;
  const int32_t* qo_indptr;
  const uint16_t* q;
  uint16_t* o;
  const char* plan;
  PlanLayout layout;
  float* ws_acc;           // [runs][2][HG][G][d] (runs x HG = kDecodeWaves): partial accumulators of split segments
  float* ws_ml;            // [runs][2][HG][G][2]: their running max (log2 units) and sum
  int32_t* status;
};

// records e as the thread's last HIP error and returns PKV_ERR_HIP
int hip_failed(hipError_t e);

hipError_t launch_kv_store(const StoreArgs& a, hipStream_t s);
hipError_t launch_kv_store_rope(const RopeArgs& a, hipStream_t s);
hipError_t launch_alloc_pages(const AllocArgs& a, hipStream_t s);
hipError_t launch_free_pages(const AllocArgs& a, hipStream_t s);
hipError_t launch_free_list_reset(int32_t* state, int32_t num_free, hipStream_t s);
hipError_t launch_rope_cache(const RopeCacheArgs& a, hipStream_t s);
hipError_t launch_metadata(const MetaArgs& a, hipStream_t s);
// Whether launch_metadata(a) also stores the new K/V rows (a.k_new set and a
// small batch); otherwise the caller launches kv_store after it.
bool metadata_stores_rows(const MetaArgs& a);
// build_attn_metadata_store's host checks and argument blocks, and its launches
// (the store inside the metadata launch when metadata_stores_rows, else a
// kv_store launch after it).
int prepare_metadata_store(const pkv_batch* batch, const pkv_page_table* page_table, const pkv_kv_pool* pool,
                           const int32_t* alloc_rows, int64_t num_alloc, int32_t num_qo_heads,
                           const pkv_attn_metadata* meta, const void* k_new, const void* v_new, MetaArgs* a,
                           StoreArgs* st);
hipError_t launch_metadata_store(const MetaArgs& a, const StoreArgs& st, hipStream_t s);
// Host checks of build_attn_metadata's arguments and its kernel argument block
// (no padding).  Returns a PKV_* code.
int prepare_metadata(const pkv_batch* batch, const pkv_page_table* page_table, int32_t page_size,
                     int64_t num_pool_rows, const int32_t* alloc_rows, int64_t num_alloc, int32_t num_qo_heads,
                     int32_t num_kv_heads, const pkv_attn_metadata* meta, MetaArgs* a);
// The plan kernel's launch as a graph kernel node: func, grid and block, and
// kernelParams pointing at *args (which must outlive the use of *p); *args is
// `a` as launch_metadata passes it.
void metadata_plan_node(const MetaArgs& a, MetaArgs* args, void** argv, hipKernelNodeParams* p);
hipError_t launch_decode(const AttnArgs& a, hipStream_t s);
hipError_t launch_extend(const AttnArgs& a, hipStream_t s);

}  // namespace pkv
