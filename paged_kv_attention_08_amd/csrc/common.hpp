// Internal definitions shared by the gfx950 kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

// ---- vector types -----------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kHeadDim = 128;
constexpr int kMaxGroup = 16;            // query heads per KV head handled by one MFMA column block
constexpr int kDecodeTargetItems = 768;  // decode split-K items the plan aims for (see plan_kernel)
constexpr int kExtendRows = 256;         // (token, query-head) rows per extend workgroup
constexpr int kPlanHeaderInts = 16;

// ---- plan layout (host and device agree through these offsets) --------------
// header (int32[16]):
//   [0] decode items written   [1] decode chunk (keys)   [2] extend tiles written
//   [3] extend tile tokens     [4] decode capacity        [5] extend capacity
// decode items   : int4 [cap_items]  (request, key begin, key end, items of that request)
// req_item_ptr   : int32 [B + 1]     first decode item of each request
// extend tiles   : int2 [cap_tiles]  (request, first new-token offset)
// alloc_ptr      : int32 [B + 1]     first alloc_rows entry of each request
struct PlanLayout {
  int64_t items_off, req_items_off, tiles_off, alloc_ptr_off, total;
  int32_t cap_items, cap_tiles, tile_q, kv_groups;
};

__host__ __device__ inline int64_t align_up64(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline int32_t extend_tile_tokens(int32_t group) { return kExtendRows / group; }

constexpr int kDecodeHeadsPerGroup = 4;  // KV heads per decode workgroup

__host__ inline PlanLayout plan_layout(int32_t max_reqs, int64_t max_tokens, int32_t group, int32_t num_kv_heads) {
  PlanLayout L;
  L.kv_groups = (num_kv_heads + kDecodeHeadsPerGroup - 1) / kDecodeHeadsPerGroup;
  const int32_t tq = extend_tile_tokens(group);
  L.tile_q = tq;
  L.cap_items = max_reqs + kDecodeTargetItems;
  const int64_t tiles = (max_tokens + tq - 1) / tq + max_reqs;
  L.cap_tiles = (int32_t)(tiles > 0 ? tiles : 1);
  int64_t off = kPlanHeaderInts * 4;
  L.items_off = off;       off += (int64_t)L.cap_items * 16;
  L.req_items_off = off;   off = align_up64(off + (int64_t)(max_reqs + 1) * 4, 16);
  L.tiles_off = off;       off += (int64_t)L.cap_tiles * 8;
  L.alloc_ptr_off = off;   off = align_up64(off + (int64_t)(max_reqs + 1) * 4, 16);
  L.total = off;
  return L;
}

// ---- device helpers ---------------------------------------------------------
__device__ inline void raise_status(int32_t* status, int32_t bits) {
  if (status) atomicOr(status, bits);
}

__device__ inline float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// fp32 -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ inline T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace pkv
