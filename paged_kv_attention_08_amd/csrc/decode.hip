// paged_decode_attn: split-K ("flash-decoding") attention of one new token per
// request over K/V rows gathered through the page table.
//
// mini-sglang learning notes, kernel passage: decode is memory bound, its cost
// is the gather of variable-length K/V, and it is parallelised across the KV
// sequence.  Deep dive 5.2: online softmax keeps a running max and sum so no
// score vector is stored.
//
// Work decomposition (from the plan written by build_attn_metadata):
//   item = (request, key range [k0, k1)); a workgroup of 4 wavefronts takes
//   one item and 4 KV heads, one wavefront per KV head.  A wavefront walks its
//   key range in tiles of 32 keys.
//
// Per tile and wavefront (lane = 16 * grp + lo):
//   * lanes 0..31 read the 32 page-table entries (requested two tiles ahead);
//     rows are broadcast with lane shuffles.  Each 16-lane group then loads
//     one whole 256-byte head row of K and of V per instruction (4 rows per
//     instruction, 8 + 8 loads per lane).  All loads are unconditional: a
//     missing key reads pool row 0 and is masked.
//   * software pipelining with one buffer: the tile's rows are written from
//     registers to the wavefront's row-major K and V tiles in LDS, which frees
//     the registers, and the next tile's loads are issued before this tile is
//     computed (a wavefront's LDS operations complete in order, so the next
//     write cannot overtake this tile's reads).
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (keys x heads): the K operand
//     (key lo (+16), 32 dims per lane group) is read from the LDS tile; the G
//     query heads of the KV head, zero-padded to 16 columns, are the B
//     operand.  Lane (grp, lo) receives keys {4 grp + v, 16 + 4 grp + v} of
//     head lo.
//   * online softmax per head: the tile max is shared by the four lane groups
//     (two cross-lane shuffles); the running max only moves when it grows by
//     more than 2^8, so the accumulator is rarely rescaled.
//   * O^T += V^T P^T on the same MFMA (d x heads, 32 keys deep): the
//     probabilities, rounded to bf16, are the B operand straight from the score
//     registers (the contraction's key order is permuted to match); the V^T
//     operand (8 keys of one dimension per lane) is read from the row-major V
//     tile with two gfx950 transpose reads (ds_read_b64_tr_b16).  No workgroup
//     barrier: each wavefront owns its tiles.
// Merge ("wavefront-reduction softmax merge"): the four lane groups hold the
// same running max, so a wavefront reduces its sums with two shuffles.  A
// request covered by one item writes its output directly; otherwise every
// item publishes its (acc, max, sum) to the workspace and a second launch
// rescales the items of each request to their common max in one pass.
// (Merging inside the first launch would need device-scope fences, which on
// this chip write back and invalidate a whole L2 per workgroup; the launch
// boundary orders the two kernels for free.)
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kTileKeys = 32;
constexpr int kWaves = kDecodeHeadsPerGroup;  // KV heads per workgroup (one per wavefront)
constexpr int kKsPitch = 136;  // bf16 per K row in LDS: 68 dwords, 16 rows x 4 dwords hit 64 distinct banks
constexpr int kVsPitch = 144;  // bf16 per V row in LDS: 72 dwords, 8 rows x 8 dwords hit 64 distinct banks

typedef short v4s __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

__device__ inline u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
// K/V rows are read once per call: stream them (whole 256-byte rows per
// instruction; with that access shape the hint measured faster than plain loads)
__device__ inline u32x4 load16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__global__ void __launch_bounds__(256, 2) decode_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[kWaves][kTileKeys * kKsPitch];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kWaves][kTileKeys * kVsPitch];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15;
  const int grp = lane >> 4;
  const int32_t* header = reinterpret_cast<const int32_t*>(a.plan);
  const int item = blockIdx.x;
  if (item >= header[0]) return;  // uniform for the workgroup
  const int g = blockIdx.y * kWaves + wave;
  if (g >= a.Hkv) return;  // no workgroup barrier below: idle wavefronts may leave

  const int4 it = reinterpret_cast<const int4*>(a.plan + a.layout.items_off)[item];
  const int i = it.x, k0 = it.y, k1 = it.z, nsplit = it.w;
  const int G = a.group;
  const int64_t tok = a.qo_indptr[i];
  if (tok < 0 || tok >= a.T) {
    if (lane == 0) raise_status(a.status, PKV_STATUS_TOKEN_COUNT);
    return;
  }
  const int32_t* pt_row = a.page_table + (int64_t)a.table_idx[i] * a.W;
  // loader: load u (0..7) of lane l moves 16 bytes (dims 8 (l % 16) ..) of key
  // 4 u + l / 16: each 16-lane group reads one whole 256-byte head row
  const uint16_t* kbase = a.k_pool + (int64_t)g * kHeadDim + lo * 8;
  const uint16_t* vbase = a.v_pool + (int64_t)g * kHeadDim + lo * 8;
  const int64_t stride = a.row_stride;
  uint16_t* ktile = ks[wave];
  uint16_t* vtile = vs[wave];

  // B operand of S^T: the G query heads of KV head g (zero for padded columns)
  bf16x8 qop[4];
  {
    const uint16_t* qrow = a.q + ((tok * a.Hq) + (int64_t)g * G + lo) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (lo < G) v = load16(qrow + (grp * 4 + kk) * 8);
      qop[kk] = as_bf16x8(v);
    }
  }

  const float c = a.scale_log2;
  float m = -INFINITY;  // running max of head lo, in log2 units (same in all four lane groups)
  float lsum = 0.f;     // this lane group's part of the running sum
  f32x4 oacc[8];        // O^T block mb: dims 16 mb + 4 grp + v of head lo
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) oacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Page-table entries of keys [kt, kt + 32): every lane loads (lanes 32..63 and
  // keys past k1 re-read an in-range entry) so the load is unconditional.
  auto load_entries = [&](int kt) -> int32_t { return pt_row[min(kt + (lane & 31), k1 - 1)]; };
  // -1 marks a key past k1 or an entry outside the pool (reported)
  auto check_entries = [&](int kt, int32_t e) -> int32_t {
    const bool in_range = lane < kTileKeys && kt + lane < k1;
    if (in_range && (e < 0 || (int64_t)e >= a.num_pool_rows)) {
      raise_status(a.status, PKV_STATUS_BAD_PAGE_ROW);
      e = -1;
    }
    return in_range ? e : -1;
  };
  u32x4 kr[8], vr[8];  // the rows of the tile in flight
  auto issue = [&](int32_t e) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t row = max(__shfl(e, 4 * u + (lane >> 4), 64), 0);  // missing keys read row 0
      kr[u] = load16_stream(kbase + row * stride);
      vr[u] = load16_stream(vbase + row * stride);
    }
  };

  int32_t ent = check_entries(k0, load_entries(k0));
  issue(ent);
  uint32_t valid_next = (uint32_t)__ballot(ent >= 0);  // bit k: key k of the tile has a row
  int32_t ent_raw = (k0 + kTileKeys < k1) ? load_entries(k0 + kTileKeys) : -1;
  for (int kt = k0; kt < k1; kt += kTileKeys) {
    const uint32_t valid = valid_next;
    // this tile's rows -> the wavefront's row-major LDS tiles (a missing key's V is zeroed)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = 4 * u + (lane >> 4);
      if (!((valid >> key) & 1u)) vr[u] = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&ktile[key * kKsPitch + lo * 8]) = kr[u];
      *reinterpret_cast<u32x4*>(&vtile[key * kVsPitch + lo * 8]) = vr[u];
    }
    // the next tile's rows go out now and stay in flight while this one is computed
    if (kt + kTileKeys < k1) {
      ent = check_entries(kt + kTileKeys, ent_raw);
      issue(ent);
      valid_next = (uint32_t)__ballot(ent >= 0);
      if (kt + 2 * kTileKeys < k1) ent_raw = load_entries(kt + 2 * kTileKeys);
    }

    // S^T (16 keys x 16 heads) per half tile; K operand: key 16 b + lo, dims (4 grp + kk) * 8
    f32x4 sc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 kop = *reinterpret_cast<const u32x4*>(&ktile[(16 * b + lo) * kKsPitch + (grp * 4 + kk) * 8]);
        sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop), qop[kk], sc[b], 0, 0, 0);
      }
    }
    // lane (grp, lo) holds keys 16 b + 4 grp + v of head lo
    float tmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (!((valid >> (16 * b + 4 * grp + v)) & 1u)) sc[b][v] = -INFINITY;
        tmax = fmaxf(tmax, sc[b][v]);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32)) * c;  // scale > 0 keeps the order
    const bool upd = tmax > m + 8.f;
    float alpha = 1.f;
    if (upd) {
      alpha = fast_exp2(m - tmax);
      m = tmax;
    }
    if (__ballot(upd) != 0) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) oacc[mb] *= alpha;
    }
    const float nms = (m == -INFINITY) ? 0.f : -m;
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[b][v] = fast_exp2(__builtin_fmaf(sc[b][v], c, nms));
        psum += p[b][v];
      }
    lsum = lsum * alpha + psum;

    // B operand: slots 0..3 keys 4 grp + 0..3, slots 4..7 keys 16 + 4 grp + 0..3
    const bf16x8 pop = as_bf16x8(u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                       pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])});
    // A operand V^T (dims 16 mb + lo, the same 8 keys): in each 16-lane group,
    // lane lo addresses 4 dims of key 4 grp + lo / 4 (then 16 + ...) and
    // receives dim lo of those 4 keys.
    const uint16_t* vrd = &vtile[(4 * grp + (lo >> 2)) * kVsPitch + 4 * (lo & 3)];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vrd + 16 * mb));
      const v4s r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(vrd + 16 * kVsPitch + 16 * mb));
      const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, oacc[mb], 0, 0, 0);
    }
  }

  // the four lane groups share the max: only the sums need reducing
  float L = lsum;
  L += shfl_xor(L, 16);
  L += shfl_xor(L, 32);
  if (lo >= G) return;
  const int64_t hq = (int64_t)g * G + lo;
  if (nsplit == 1) {  // the whole request in one item: normalise and write
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* orow = a.o + (tok * a.Hq + hq) * kHeadDim + 4 * grp;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      *reinterpret_cast<uint2*>(orow + 16 * mb) =
          make_uint2(pack_bf16x2(oacc[mb][0] * inv, oacc[mb][1] * inv), pack_bf16x2(oacc[mb][2] * inv, oacc[mb][3] * inv));
    return;
  }
  // several items: publish this item's (acc, max, sum) for the merge launch
  float* dst = a.ws_acc + ((int64_t)item * a.Hq + hq) * kHeadDim + 4 * grp;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
    *reinterpret_cast<float4*>(dst + 16 * mb) = make_float4(oacc[mb][0], oacc[mb][1], oacc[mb][2], oacc[mb][3]);
  if (grp == 0) *reinterpret_cast<float2*>(a.ws_ml + ((int64_t)item * a.Hq + hq) * 2) = make_float2(m, L);
}

// One workgroup per (request, pair of query heads), one thread per dimension:
// a single pass over the request's items with a running max; the loads of an
// item do not depend on the running state, so consecutive items overlap.
__global__ void __launch_bounds__(256) decode_merge_kernel(AttnArgs a) {
  const int i = blockIdx.x;
  const int hq = blockIdx.y * 2 + (threadIdx.x >> 7);
  const int d = threadIdx.x & 127;
  if (hq >= a.Hq) return;
  const int32_t* req_items = reinterpret_cast<const int32_t*>(a.plan + a.layout.req_items_off);
  const int j0 = req_items[i];
  const int j1 = req_items[i + 1];
  if (j1 - j0 <= 1) return;  // written by the first launch
  const int64_t tok = a.qo_indptr[i];
  if (tok < 0 || tok >= a.T) return;
  float Mx = -INFINITY, den = 0.f, num = 0.f;
#pragma unroll 4
  for (int j = j0; j < j1; ++j) {
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + ((int64_t)j * a.Hq + hq) * 2);
    const float aj = a.ws_acc[((int64_t)j * a.Hq + hq) * kHeadDim + d];
    const float Mn = fmaxf(Mx, ml.x);
    const float so = (Mx == -INFINITY) ? 0.f : fast_exp2(Mx - Mn);
    const float sn = (ml.x == -INFINITY) ? 0.f : fast_exp2(ml.x - Mn);
    den = den * so + ml.y * sn;
    num = num * so + aj * sn;
    Mx = Mn;
  }
  const float r = den > 0.f ? num / den : 0.f;
  const __bf16 ob = (__bf16)r;
  a.o[(tok * a.Hq + hq) * kHeadDim + d] = __builtin_bit_cast(uint16_t, ob);
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, hipStream_t s) {
  if (a.num_decode == 0) return hipSuccess;
  const dim3 grid((unsigned)a.layout.cap_items, (unsigned)a.layout.kv_groups);
  hipLaunchKernelGGL(decode_kernel, grid, dim3(64 * kWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)a.num_decode, (unsigned)((a.Hq + 1) / 2)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
