// kv_store_rope and its rotary table: rotary position embedding (with an
// optional per-head RMS norm) applied to q and k while k and v are scattered to
// the pool.
//
// mini-sglang architecture deep dive, section 7.2: the attention layer
// normalises q and k per head when the model asks for it (Qwen3), rotates
// them by position, and the backend then stores K/V and attends.  Section 7.3:
// rotary_dim equals head_size, the inverse frequencies are
// base^(-2i/rotary_dim), and the rotation is applied in place from a cos/sin
// table indexed by position.  Fusing it into the store reads k and v once and
// writes the pool once; q is rotated in the same pass.
//
// Layout: a workgroup (256 threads = 16 groups of 16 lanes) takes 16 head rows
// of one token, so a token of Hq + 2 Hkv rows spreads over several workgroups
// and a decode batch of a few hundred tokens still fills the chip; a 16-lane
// group takes one 128-element head row, lane i holding elements
// 4i..4i+3 and 64+4i..64+4i+3, i.e. the rotation pairs (j, j + 64) sit in the
// same lane.  Rows Hq q heads, then Hkv k heads, then Hkv v heads (copied).
// The norm's sum of squares is reduced over the 16 lanes with shuffles.
// Everything is HBM traffic: per token q is read and written, k and v read,
// two pool rows written, plus one 512-byte table row.
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kGroups = 16;  // head rows in flight per workgroup
// below this many tokens (two workgroups per CU on 256 CUs) tokens are split
// into 16-row chunks
constexpr int kSplitBelowTokens = 512;

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ inline uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }

__device__ inline void unpack4(uint2 v, float* x) {
  x[0] = bf16_to_f32(v.x & 0xFFFF);
  x[1] = bf16_to_f32(v.x >> 16);
  x[2] = bf16_to_f32(v.y & 0xFFFF);
  x[3] = bf16_to_f32(v.y >> 16);
}

// Work item = (token t, chunk c): the chunk's 16 groups take head rows
// c * chunk_rows .. (c + 1) * chunk_rows - 1 of token t, a group stepping by 16
// rows.  With one chunk per token a workgroup does the whole token; small
// batches split tokens into 16-row chunks so the grid still fills the chip.
// Items run chunk-major (item = c * T + t), so a token's chunks land on the
// same XCD when T is a multiple of 8 and share its table row in that XCD's L2.
// The table row is read once per item, before the row loop.
__global__ void __launch_bounds__(256) kv_store_rope_kernel(RopeArgs a, int chunks, int chunk_rows) {
  const int lane16 = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const int nrows = a.Hq + 2 * a.Hkv;
  const int64_t items = a.num_tokens * chunks;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    int c = 0;
    int64_t t = item;
    if (chunks > 1) {
      c = (int)(item / a.num_tokens);
      t = item - (int64_t)c * a.num_tokens;
    }
    const int32_t pos = a.positions[t];
    // -1 marks a token build_attn_metadata could not map (already reported)
    if (pos < 0 || pos >= a.max_position) {
      if (c == 0 && threadIdx.x == 0 && pos != -1) raise_status(a.status, PKV_STATUS_BAD_POSITION);
      continue;  // uniform for the workgroup
    }
    const int32_t loc = a.out_loc[t];
    const bool store = loc >= 0 && (int64_t)loc < a.num_rows;
    if (!store && c == 0 && threadIdx.x == 0 && loc != -1) raise_status(a.status, PKV_STATUS_BAD_OUT_LOC);
    const float* cs = a.cos_sin + (int64_t)pos * kHeadDim;
    const float4 c4 = *reinterpret_cast<const float4*>(cs + 4 * lane16);
    const float4 s4 = *reinterpret_cast<const float4*>(cs + kHeadDim / 2 + 4 * lane16);
    const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
    const float ss[4] = {s4.x, s4.y, s4.z, s4.w};
    const int r_end = min(nrows, (c + 1) * chunk_rows);
    for (int r = c * chunk_rows + grp; r < r_end; r += kGroups) {
      const uint16_t* src;
      uint16_t* dst;
      const uint16_t* w = nullptr;
      bool rotate = true;
      if (r < a.Hq) {
        dst = a.q + (t * a.Hq + r) * kHeadDim;
        src = dst;
        w = a.q_weight;
      } else if (r < a.Hq + a.Hkv) {
        const int g = r - a.Hq;
        src = a.k_new + (t * a.Hkv + g) * kHeadDim;
        dst = store ? a.k_pool + (int64_t)loc * a.row_stride + g * kHeadDim : nullptr;
        w = a.k_weight;
      } else {
        const int g = r - a.Hq - a.Hkv;
        src = a.v_new + (t * a.Hkv + g) * kHeadDim;
        dst = store ? a.v_pool + (int64_t)loc * a.row_stride + g * kHeadDim : nullptr;
        rotate = false;
      }
      // uniform per 16-lane group: r is the same for all of its lanes
      const uint2 lo = *reinterpret_cast<const uint2*>(src + 4 * lane16);
      const uint2 hi = *reinterpret_cast<const uint2*>(src + kHeadDim / 2 + 4 * lane16);
      uint2 olo = lo, ohi = hi;
      if (rotate) {
        float x1[4], x2[4];
        unpack4(lo, x1);
        unpack4(hi, x2);
        if (w) {
          float sq = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) sq += x1[e] * x1[e] + x2[e] * x2[e];
#pragma unroll
          for (int m = 8; m >= 1; m >>= 1) sq += __shfl_xor(sq, m, 64);  // stays inside the 16-lane group
          const float inv = 1.0f / sqrtf(sq * (1.0f / kHeadDim) + a.eps);
          float w1[4], w2[4];
          unpack4(*reinterpret_cast<const uint2*>(w + 4 * lane16), w1);
          unpack4(*reinterpret_cast<const uint2*>(w + kHeadDim / 2 + 4 * lane16), w2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x1[e] = x1[e] * inv * w1[e];
            x2[e] = x2[e] * inv * w2[e];
          }
        }
        float y1[4], y2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y1[e] = __builtin_fmaf(x1[e], cc[e], -x2[e] * ss[e]);
          y2[e] = __builtin_fmaf(x2[e], cc[e], x1[e] * ss[e]);
        }
        olo = make_uint2(pack2(y1[0], y1[1]), pack2(y1[2], y1[3]));
        ohi = make_uint2(pack2(y2[0], y2[1]), pack2(y2[2], y2[3]));
      }
      if (dst) {
        *reinterpret_cast<uint2*>(dst + 4 * lane16) = olo;
        *reinterpret_cast<uint2*>(dst + kHeadDim / 2 + 4 * lane16) = ohi;
      }
    }
  }
}

// one thread per (position, frequency)
__global__ void __launch_bounds__(256) rope_cache_kernel(RopeCacheArgs a) {
  const int64_t n = (int64_t)a.max_position * (kHeadDim / 2);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = idx / (kHeadDim / 2);
    const int i = (int)(idx - p * (kHeadDim / 2));
    // theta_i = base^(-2i/d) = 2^(-(2i/d) log2(base))
    const double theta = exp2(-(2.0 * i / kHeadDim) * a.log2_base);
    double sn, cn;
    sincos((double)p * theta, &sn, &cn);
    a.cache[p * kHeadDim + i] = (float)cn;
    a.cache[p * kHeadDim + kHeadDim / 2 + i] = (float)sn;
  }
}

}  // namespace

hipError_t launch_kv_store_rope(const RopeArgs& a, hipStream_t s) {
  // whole tokens per workgroup once the tokens alone give every CU two
  // workgroups; below that, 16-row chunks (measured with 48 rows per token:
  // chunks 15% faster at 256 tokens, 9% slower at 1024)
  const int nchunks = (a.Hq + 2 * a.Hkv + kGroups - 1) / kGroups;
  const bool split = a.num_tokens < kSplitBelowTokens;
  const int chunks = split ? nchunks : 1;
  const int chunk_rows = split ? kGroups : nchunks * kGroups;
  int64_t blocks = a.num_tokens * chunks;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(kv_store_rope_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, chunks, chunk_rows);
  return hipGetLastError();
}

hipError_t launch_rope_cache(const RopeCacheArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.max_position * (kHeadDim / 2);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(rope_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
