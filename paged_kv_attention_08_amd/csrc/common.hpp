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
constexpr int kDecodeTileKeys = 32;      // keys per decode tile
constexpr int kDecodeWaves = 2048;       // persistent decode wavefronts (256 CUs x 8)
constexpr int kDecodeWgWaves = 8;        // wavefronts per decode workgroup
constexpr int kExtendRows = 256;         // (token, query-head) rows per extend workgroup
constexpr int kPlanHeaderInts = 16;

// ---- plan layout (host and device agree through these offsets) --------------
// header (int32[16]):
//   [0] decode tiles in the flat order (KV-head groups x sum of the decode
//       requests' tiles)
//   [1] decode tiles per run           [2] extend tiles written
//   [3] extend tile tokens             [4] decode runs with work
//   [5] extend capacity
// dec_tile_ptr   : int32 [B + 1]     first decode tile of each request (per KV head;
//                                    0 tiles for extend and invalid requests)
// extend tiles   : int2 [cap_tiles]  (request, first new-token offset), most keys first
// tiles_raw      : int2 [cap_tiles]  the same, request by request (sort input)
// alloc_ptr      : int32 [B + 1]     first alloc_rows entry of each request
// The flat decode order is request-major, then group of HG KV heads, then key
// tile: with Hg = Hkv / HG groups (HG = decode_heads_per_group(Hkv)), the
// tiles of (request i, group gg) are Hg * dec_tile_ptr[i] + gg * n_i + [0, n_i).
struct PlanLayout {
  int64_t dec_tiles_off, tiles_off, tiles_raw_off, alloc_ptr_off, total;
  int32_t cap_tiles, tile_q;
};

__host__ __device__ inline int64_t align_up64(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline int32_t extend_tile_tokens(int32_t group) { return kExtendRows / group; }

__host__ inline PlanLayout plan_layout(int32_t max_reqs, int64_t max_tokens, int32_t group, int32_t num_kv_heads) {
  (void)num_kv_heads;
  PlanLayout L;
  const int32_t tq = extend_tile_tokens(group);
  L.tile_q = tq;
  const int64_t tiles = (max_tokens + tq - 1) / tq + max_reqs;
  L.cap_tiles = (int32_t)(tiles > 0 ? tiles : 1);
  int64_t off = kPlanHeaderInts * 4;
  L.dec_tiles_off = off;   off = align_up64(off + (int64_t)(max_reqs + 1) * 4, 16);
  L.tiles_off = off;       off += (int64_t)L.cap_tiles * 8;
  L.tiles_raw_off = off;   off += (int64_t)L.cap_tiles * 8;
  L.alloc_ptr_off = off;   off = align_up64(off + (int64_t)(max_reqs + 1) * 4, 16);
  L.total = off;
  return L;
}

// KV heads a decode run reads together (one wavefront each): the largest of
// 8, 4, 2, 1 that divides Hkv, so that no wavefront idles.  A run is HG
// wavefronts walking the same tiles; there are kDecodeWaves / HG runs.
__host__ __device__ inline int32_t decode_heads_per_group(int32_t num_kv_heads) {
  return num_kv_heads % 8 == 0 ? 8 : num_kv_heads % 4 == 0 ? 4 : num_kv_heads % 2 == 0 ? 2 : 1;
}

// Decode workspace: per wavefront (a run and one KV head of its group) two
// partial states (the piece of the segment the run starts inside and of the
// one it ends inside), each G query heads x
// (head_dim fp32 accumulator + running max + running sum).
__host__ __device__ constexpr int64_t decode_ws_floats(int32_t max_group) {
  return (int64_t)kDecodeWaves * 2 * max_group * (kHeadDim + 2);
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
