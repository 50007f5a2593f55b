// paged_extend_attn: chunked prefill on a cached (possibly radix-shared)
// prefix, K/V gathered through the page table, bf16 MFMA for QK^T and PV.
//
// mini-sglang learning notes, Req and chunked-prefill passages: a chunk adds
// extend_len = device_len - cached_len new tokens on top of cached_len tokens
// already in the pool; prefill is compute bound and needs large tiles to keep
// the matrix units busy.  Deep dive 5.2: FlashAttention tiling with an online
// softmax keeps the n x n score matrix out of HBM.
//
// Work decomposition: one workgroup (8 wavefronts, one per 32 rows) per plan
// tile = (request, TQ consecutive new tokens) and KV head g.  Its 256 rows are
// the (token, query head) pairs of the tile that share KV head g, token-major
// (row = tq * G + query head within the group), so each gathered K/V tile is
// loaded once for all G query heads and 256 rows.  Wavefront w owns rows
// 32w..32w+31.  Workgroups are dispatched round-robin over the 8 XCDs, each
// with its own L2; the (head, tile) items are laid out so that every XCD
// takes one contiguous, request-major range of them, and the workgroups that
// re-read one request's K/V for one head (and a radix-shared prefix) meet in
// the same L2.
//
// Per 64-key tile:
//   * the workgroup gathers 64 K rows and 64 V rows of head g into registers
//     two tiles ahead (two register sets, page-table entries one tile before
//     that): wavefront w takes keys 8w..8w+7, each 16-lane group one whole
//     256-byte head row per load (16 bytes per lane), so a load instruction
//     touches 4 rows.  (With one key per lane, every instruction touched 64
//     scattered rows and half the address translations missed the per-CU
//     TLB.)  Both tiles are stored row-major ([key][d]) in LDS as contiguous
//     256-byte runs, in two stages: tile n + 1 is stored while tile n is in
//     use, so one barrier per tile suffices;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys x rows): the K operand
//     is read from LDS, Q stays in registers for the whole loop.  In the
//     32x32 accumulator layout each lane owns one row (query) and 16 of its 32
//     keys, so the row max needs one cross-half shuffle;
//   * causal masking is applied only on tiles that reach past the first
//     row's position; prefix tiles run unmasked;
//   * online softmax in fp32 without a per-tile max pass: probabilities are
//     taken against the running max and a lane's sum of them (computed anyway
//     for the normaliser) detects growth past 2^64, after which the tile is
//     redone against its true max (the first tile always is);
//   * O^T += V^T P^T: the probabilities, rounded to bf16, are used as the B
//     operand straight from the score accumulator registers (the key order of
//     the contraction is permuted to match them); the V^T operand (8 keys of
//     one d per lane) comes from the row-major V tile through two gfx950 LDS
//     transpose reads (ds_read_b64_tr_b16): in each 16-lane group, lane j
//     addresses 4 dims of key (j / 4) and lane i receives dim i of 4 keys.
#include <type_traits>

#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kKeyTile = 64;
constexpr int kVW = 4;  // V^T operand reads in flight ahead of the PV MFMAs
constexpr int kKsStride = 136;  // bf16 elements per K row in LDS (128 + 8 pad)
constexpr int kVsStride = 160;  // bf16 elements per V row in LDS (80 dwords: 4 rows x 16 dwords hit 64 distinct banks)
constexpr int kWaves = 8;
static_assert(kExtendRows == 32 * kWaves, "one 32-row block per wavefront");
constexpr int kWaveKeys = kKeyTile / kWaves;  // keys of a tile one wavefront gathers
constexpr int kLoads = kWaveKeys / 4;         // 16-byte loads per lane per tile and per K / V (4 rows per load)

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ inline float dot2_bf16(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w), __builtin_bit_cast(bf16x2v, 0x3F803F80u), acc, false);
}

__global__ void __launch_bounds__(64 * kWaves, 8 / kWaves) extend_kernel(AttnArgs a) {
  // two LDS stages: tile n lives in stage n % 2
  __shared__ __attribute__((aligned(16))) uint16_t ks_all[2][kKeyTile * kKsStride];
  __shared__ __attribute__((aligned(16))) uint16_t vs_all[2][kKeyTile * kVsStride];

  const int32_t* header = reinterpret_cast<const int32_t*>(a.plan);
  // Workgroups are dispatched to the 8 XCDs round-robin (linear id % 8) and
  // each XCD has its own L2.  Give every XCD one contiguous range of the
  // (KV head, tile) items, tiles request-major as the plan lists them, so the
  // workgroups that re-read one request's K/V for one head share an L2.
  const int n_tiles = header[2];
  const int n_items = n_tiles * a.Hkv;
  const int per_xcd = (n_items + 7) / 8;
  const int xcd = blockIdx.x & 7;
  const int slot_in_xcd = blockIdx.x >> 3;
  if (slot_in_xcd >= per_xcd) return;  // uniform for the workgroup
  const int item = xcd * per_xcd + slot_in_xcd;
  if (item >= n_items) return;
  const int g = item / n_tiles;
  const int tile = item - g * n_tiles;

  const int2 tl = reinterpret_cast<const int2*>(a.plan + a.layout.tiles_off)[tile];
  const int i = tl.x;
  const int t0 = tl.y;
  const int32_t c = a.cached_len[i];
  const int32_t dl = a.device_len[i];
  const int64_t tokbase = a.qo_indptr[i];
  const int G = a.group;
  const int TQ = a.layout.tile_q;
  const int n_tok = min(TQ, dl - c - t0);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int row = wave * 32 + l32;
  const int tq = row / G;
  const int gh = row - tq * G;
  const int64_t token = tokbase + t0 + tq;
  const bool row_valid = (tq < n_tok) && token >= 0 && token < a.T;
  // a row past the tile's tokens sees every key (its q is zero and it is
  // never written), so its running max is finite after the first tile
  const int pos = row_valid ? c + t0 + tq : 0x7fffffff;
  const int h = g * G + gh;

  bf16x8 qop[8];
  {
    const uint16_t* qrow = a.q + (token * a.Hq + h) * kHeadDim + half * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qop[kk] = as_bf16x8(row_valid ? load16(qrow + 16 * kk) : make_uint4(0, 0, 0, 0));
  }

  const int kv_end = min(dl, c + t0 + n_tok);
  const int32_t* pt_row = a.page_table + (int64_t)a.table_idx[i] * a.W;
  const uint16_t* kbase = a.k_pool + (int64_t)g * kHeadDim + (lane & 15) * 8;
  const uint16_t* vbase = a.v_pool + (int64_t)g * kHeadDim + (lane & 15) * 8;
  const uint32_t row_elems = (uint32_t)a.row_stride;  // < 2^31, checked on the host
  const uint32_t n_rows = (uint32_t)a.num_pool_rows;

  // loader: load u (0..kLoads-1) of lane l in wavefront w moves 16 bytes
  // (dims 8 (l % 16) ..) of key kWaveKeys w + 4 u + l / 16 of the tile.  Keys past kv_end
  // re-read the last valid key's row: finite data, and such keys only occur in the
  // last tile, which is always masked, so their probabilities are exactly 0.  Tiles
  // past the end are gathered the same way: every tile issues the same loads, which
  // lets the compiler wait only for the loads of the tile being stored (with
  // conditional gathers it waited for the previous tile's loads as well, halving
  // the prefetch distance).
  uint4 kpre[2][kLoads], vpre[2][kLoads];  // [register set][load]
  // page-table entries of the next tile to gather, one per load (16 lanes share one)
  int32_t ent[kLoads];
  auto load_entries = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) ent[u] = pt_row[min(kt + kWaveKeys * wave + 4 * u + (lane >> 4), kv_end - 1)];
  };
  auto gather = [&](int kt, auto set_tag) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value;
    uint32_t r[kLoads];
    bool bad = false;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      r[u] = (uint32_t)ent[u];
      const bool b = r[u] >= n_rows;  // also catches negative entries
      bad |= b;
      r[u] = b ? 0u : r[u];
    }
    // the next tile's entries are requested before this tile's rows, so the
    // wait for them (one tile later) can leave these row loads in flight
    load_entries(kt + kKeyTile);
    // 32 x 32 -> 64-bit row offsets
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const uint64_t off = (uint64_t)r[u] * row_elems;
      kpre[SET][u] = load16(kbase + off);
      vpre[SET][u] = load16(vbase + off);
    }
    if (bad) raise_status(a.status, PKV_STATUS_BAD_PAGE_ROW);
  };

  f32x16 oacc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[nb][v] = 0.f;
  float m = -INFINITY;
  float lsum = 0.f;
  const float csc = a.scale_log2;
  const int min_pos = c + t0;
  // tiles whose keys all lie at or before the first row's position need no mask
  const int kt_mask = min(kv_end, ((min_pos + 1) / kKeyTile) * kKeyTile);

  // tile kt from register set S into LDS stage S
  auto store_tile = [&](int kt, auto set_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(set_tag)::value;
    (void)kt;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int key = kWaveKeys * wave + 4 * u + (lane >> 4);
      *reinterpret_cast<uint4*>(&ks_all[S][key * kKsStride + (lane & 15) * 8]) = kpre[S][u];
      *reinterpret_cast<uint4*>(&vs_all[S][key * kVsStride + (lane & 15) * 8]) = vpre[S][u];
    }
  };
  // One 64-key tile in stage SET.  MASK: the tile reaches past the first
  // row's position, so keys beyond a row's own position are masked (diagonal
  // and ragged end).
  auto key_tile = [&](int kt, auto set_tag) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value;
    const bool MASK = kt >= kt_mask;  // uniform
    const uint16_t* ks = ks_all[SET];
    const uint16_t* vs = vs_all[SET];

    // S^T = K Q^T : two 32-key blocks (raw scores, scale folded into exp below);
    // the two accumulation chains alternate and the K operands are read from
    // LDS four MFMAs ahead, the first four before the next tile's store and
    // gathers.  sched_barrier pins that order: left to itself the compiler
    // issued each read about one MFMA before its use and every MFMA waited
    // for the LDS latency (3.7% of the launch on the shared-prefix batch).
    f32x16 sacc[2];
    auto kread = [&](int j) __attribute__((always_inline)) {
      return as_bf16x8(*reinterpret_cast<const uint4*>(&ks[((j & 1) * 32 + l32) * kKsStride + half * 8 + 16 * (j >> 1)]));
    };
    bf16x8 kb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j] = kread(j);
    __builtin_amdgcn_sched_barrier(0);
    // the next tile goes to the other stage (last read before the previous
    // barrier); its register set then receives the tile three ahead
    store_tile(kt + kKeyTile, std::integral_constant<int, SET ^ 1>{});
    gather(kt + 3 * kKeyTile, std::integral_constant<int, SET ^ 1>{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int mb = j & 1, kk = j >> 1;
      sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[j & 3], qop[kk], kk == 0 ? f32x16{} : sacc[mb], 0, 0, 0);
      if (j + 4 < 16) kb[j & 3] = kread(j + 4);
      __builtin_amdgcn_sched_barrier(0);
    }
    // element v of block mb is key kt + 32 mb + 8 (v / 4) + 4 half + v % 4 of row l32
    if (MASK) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kt + 32 * mb + 8 * (v >> 2) + 4 * half + (v & 3) > pos) sacc[mb][v] = -INFINITY;
    }
    // Probabilities against the running max m without a max pass: p =
    // exp2(s c - m), rounded to bf16 (the PV operand), and this lane's sum of
    // its 32 of them.  A lane's sum bounds each of its p, so while every sum
    // stays at or below 2^64 (and finite) nothing can overflow: fp32 and bf16
    // keep their relative precision at any such magnitude, and the output is
    // normalised by the same sum of bf16 values.  The first tile (m = -inf) and
    // a tile whose scores grew by more than 64 (log2 units) since the last max
    // take the slow path: the true tile max (both lane halves of a row), the
    // rescale of the accumulator and sum, and the probabilities again.
    // V^T operand of PV MFMA m (numbered below): slots 0..3 are keys key0 +
    // 0..3, slots 4..7 keys key0 + 8..11.  The first kVW are read before the
    // softmax, so their latency is hidden behind it.
    auto vread = [&](int m) __attribute__((always_inline)) {
      const int mb = m >> 3, kq = (m >> 2) & 1, nb = m & 3;
      const int key0 = mb * 32 + 16 * kq + 4 * half;
      const int j16 = lane & 15;
      const uint16_t* vp = &vs[(key0 + (j16 >> 2)) * kVsStride + nb * 32 + ((lane >> 4) & 1) * 16 + 4 * (j16 & 3)];
      const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)vp);
      const v4s r2 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vp + 8 * kVsStride));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vb[kVW];
#pragma unroll
    for (int m = 0; m < kVW; ++m) vb[m] = vread(m);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t pk[2][8];  // bf16 pairs: block mb, words 4 kq + 0..3
    float psum0, psum1;
    auto make_p = [&](float nms) __attribute__((always_inline)) {
      psum0 = 0.f;
      psum1 = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const float p0 = fast_exp2(__builtin_fmaf(sacc[mb][2 * w], csc, nms));
          const float p1 = fast_exp2(__builtin_fmaf(sacc[mb][2 * w + 1], csc, nms));
          pk[mb][w] = pack_bf16x2(p0, p1);
          if (w & 1) psum1 = dot2_bf16(pk[mb][w], psum1);
          else psum0 = dot2_bf16(pk[mb][w], psum0);
        }
    };
    float alpha = 1.f;
    bool slow = __ballot(m == -INFINITY) != 0;
    if (!slow) {
      make_p(-m);
      slow = __ballot(!(psum0 + psum1 <= 0x1p64f)) != 0;
    }
    if (slow) {
      float tmax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[mb][v]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * csc;  // scale > 0 keeps the order
      const float mn = fmaxf(m, tmax);
      alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
      m = mn;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[nb][v] *= alpha;
      make_p(m == -INFINITY ? 0.f : -m);
    }

    // O^T += V^T P^T, 16 keys per MFMA: MFMA m = 4 (2 mb + kq) + nb; its V^T
    // operand is read kVW MFMAs ahead, in an order pinned as for S
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int mb = m >> 3, kq = (m >> 2) & 1, nb = m & 3;
      const bf16x8 pop = as_bf16x8(make_uint4(pk[mb][4 * kq], pk[mb][4 * kq + 1], pk[mb][4 * kq + 2], pk[mb][4 * kq + 3]));
      oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[m % kVW], pop, oacc[nb], 0, 0, 0);
      if (m + kVW < 16) vb[m % kVW] = vread(m + kVW);
      __builtin_amdgcn_sched_barrier(0);
    }
    lsum = lsum * alpha + (psum0 + psum1);
  };

  load_entries(0);
  gather(0, std::integral_constant<int, 0>{});
  gather(kKeyTile, std::integral_constant<int, 1>{});
  store_tile(0, std::integral_constant<int, 0>{});
  gather(2 * kKeyTile, std::integral_constant<int, 0>{});
  __syncthreads();
  // both tiles of a pair always run, so every path into a tile has the same
  // loads in flight (an odd last tile runs after the loop)
  int kt = 0;
  for (; kt + kKeyTile < kv_end; kt += 2 * kKeyTile) {
    key_tile(kt, std::integral_constant<int, 0>{});
    __syncthreads();
    key_tile(kt + kKeyTile, std::integral_constant<int, 1>{});
    __syncthreads();
  }
  if (kt < kv_end) {
    key_tile(kt, std::integral_constant<int, 0>{});
    __syncthreads();
  }

  const float L = lsum + __shfl_xor(lsum, 32, 64);
  if (row_valid) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* orow = a.o + (token * a.Hq + h) * kHeadDim;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = nb * 32 + 8 * q4 + 4 * half;
        uint2 out;
        out.x = pack_bf16x2(oacc[nb][4 * q4 + 0] * inv, oacc[nb][4 * q4 + 1] * inv);
        out.y = pack_bf16x2(oacc[nb][4 * q4 + 2] * inv, oacc[nb][4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = out;
      }
  }
}

}  // namespace

hipError_t launch_extend(const AttnArgs& a, hipStream_t s) {
  if (a.num_decode >= a.B) return hipSuccess;
  // one workgroup per (KV head, tile) item, rounded up to whole XCD rounds
  const int64_t n = ((int64_t)a.layout.cap_tiles * a.Hkv + 7) / 8 * 8;
  const dim3 grid((unsigned)n);
  hipLaunchKernelGGL(extend_kernel, grid, dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
