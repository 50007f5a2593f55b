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
//   * lanes 0..31 read the 32 page-table entries; rows are broadcast with
//     lane shuffles;
//   * K: lane (grp, lo) loads key lo (+16) of the tile, 4 x 16 bytes: its
//     d-chunks form the A operand of v_mfma_f32_16x16x32_bf16 directly
//     (keys x d), the G query heads of the KV head are the B operand
//     (d x heads, zero-padded to 16), so the MFMA gives S^T (keys x heads).
//     Nothing in a tile is reused by another wavefront, so K and V go from
//     HBM straight to registers in operand layout; LDS only carries the
//     probabilities between lanes.
//   * softmax: lane (grp, n) holds 8 keys of head n; each of the 4 lane
//     groups keeps its own running max / sum (merged once at the end); the
//     max only moves when it grows by more than 2^8, so the accumulator is
//     rarely rescaled (probabilities stay <= 256, exact in the final ratio);
//   * V: lane (grp, lo) loads the same 8 keys' d-chunk lo (16 bytes each);
//     probabilities are rounded to bf16 and PV runs as v_dot2 (2 keys per
//     instruction, fp32 accumulate) on key pairs built with v_perm;
//   * the page-table entries of the next tile are requested before this
//     tile's rows, so a tile waits for one memory latency; all loads are
//     unconditional (a missing key reads pool row 0 and is masked), which lets
//     the compiler wait for the K rows without waiting for the V rows.
//     (Non-temporal loads were measured slower here than plain ones.)
// Merge ("wavefront-reduction softmax merge"): each wavefront first merges
// its four lane groups with cross-lane shuffles.  A request covered by one
// item writes its output directly; otherwise every item publishes its
// (acc, max, sum) to the workspace and a second launch rescales the items of
// each request to their common max in one pass.  (Merging inside the first
// launch would need device-scope fences, which on this chip write back and
// invalidate a whole L2 per workgroup; the launch boundary orders the two
// kernels for free.)
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kTileKeys = 32;
constexpr int kWaves = kDecodeHeadsPerGroup;  // KV heads per workgroup (one per wavefront)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

__device__ inline u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int GP>
__global__ void __launch_bounds__(256, (GP >= 16 ? 1 : 2)) decode_kernel(AttnArgs a) {
  __shared__ u32x4 p_lds[kWaves][4][16];  // [wave][lane group][head] 8 probabilities as bf16 pairs
  __shared__ float x_lds[kWaves][4][16];  // [wave][lane group][head] rescale factor
  __shared__ float l_lds[kWaves][16];     // [wave][head] softmax denominator

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15;
  const int grp = lane >> 4;
  const int32_t* header = reinterpret_cast<const int32_t*>(a.plan);
  const int item = blockIdx.x;
  if (item >= header[0]) return;  // uniform for the workgroup
  const int g = blockIdx.y * kWaves + wave;
  const bool active = g < a.Hkv;  // idle wavefronts still take part in the barriers

  const int4 it = reinterpret_cast<const int4*>(a.plan + a.layout.items_off)[item];
  const int i = it.x, k0 = it.y, k1 = it.z, nsplit = it.w;
  const int G = a.group;
  const int64_t tok = a.qo_indptr[i];
  if (tok < 0 || tok >= a.T) {
    if (threadIdx.x == 0) raise_status(a.status, PKV_STATUS_TOKEN_COUNT);
    return;  // uniform: same request for the whole workgroup
  }
  const int gg = active ? g : 0;
  const int32_t* pt_row = a.page_table + (int64_t)a.table_idx[i] * a.W;
  const uint16_t* kbase = a.k_pool + (int64_t)gg * kHeadDim;
  const uint16_t* vbase = a.v_pool + (int64_t)gg * kHeadDim;
  const int64_t stride = a.row_stride;

  // B operand: the G query heads of KV head g (zero for padded columns)
  bf16x8 qop[4];
  {
    const uint16_t* qrow = a.q + ((tok * a.Hq) + (int64_t)gg * G + lo) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (active && lo < G) v = load16(qrow + (grp * 4 + kk) * 8);
      qop[kk] = as_bf16x8(v);
    }
  }

  const float c = a.scale_log2;
  float m = -INFINITY;
  float lsum = 0.f;
  float acc[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  // Entries of keys [kt, kt + 32): every lane loads (lanes 32..63 and keys past
  // k1 re-read an in-range entry) so the load is unconditional; keys past k1
  // are marked -1 afterwards with a select.
  auto load_entries = [&](int kt) -> int32_t { return pt_row[min(kt + (lane & 31), k1 - 1)]; };
  int32_t ent_next = load_entries(k0);
  for (int kt = k0; active && kt < k1; kt += kTileKeys) {
    int32_t ent = ent_next;
    // page-table entries of the next tile go out before this tile's rows
    if (kt + kTileKeys < k1) ent_next = load_entries(kt + kTileKeys);
    const bool in_range = lane < kTileKeys && kt + lane < k1;
    if (in_range && (ent < 0 || (int64_t)ent >= a.num_pool_rows)) {
      raise_status(a.status, PKV_STATUS_BAD_PAGE_ROW);
      ent = -1;
    }
    if (!in_range) ent = -1;
    const bool clean = __ballot(lane < kTileKeys && ent < 0) == 0;  // a full tile of valid rows
    // K rows of this lane: keys lo and 16 + lo of the tile
    int rk[2];
    rk[0] = __shfl(ent, lo, 64);
    rk[1] = __shfl(ent, 16 + lo, 64);
    // V rows: keys 16 * b + 4 * grp + v
    int rv[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) rv[b][v] = __shfl(ent, 16 * b + 4 * grp + v, 64);

    // unconditional loads; a missing key reads pool row 0 and is masked below
    u32x4 kr[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint16_t* kp = kbase + (int64_t)max(rk[b], 0) * stride + grp * 32;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kr[b][kk] = load16(kp + kk * 8);
    }
    u32x4 vr[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) vr[b][v] = load16(vbase + (int64_t)max(rv[b][v], 0) * stride + lo * 8);

    // S^T (16 keys x 16 heads) per half tile
    f32x4 sc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[b][kk]), qop[kk], sc[b], 0, 0, 0);
    }
    // lane (grp, lo) holds keys 16 b + 4 grp + v of head lo; those are the keys of rv[b][v]
    float sv[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float s = rv[b][v] >= 0 ? sc[b][v] * c : -INFINITY;
        sv[b][v] = s;
        tmax = fmaxf(tmax, s);
      }
    const bool upd = tmax > m + 8.f;
    float alpha = 1.f;
    if (upd) {
      alpha = fast_exp2(m - tmax);
      m = tmax;
    }
    const float ms = (m == -INFINITY) ? 0.f : m;
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[b][v] = fast_exp2(sv[b][v] - ms);
        psum += p[b][v];
      }
    lsum = lsum * alpha + psum;
    const bool any_upd = __ballot(upd) != 0;
    p_lds[wave][grp][lo] = u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                 pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
    if (any_upd) x_lds[wave][grp][lo] = alpha;

    if (!clean) {  // ragged tile: missing keys contribute exactly zero (p is 0, V forced to 0)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (rv[b][v] < 0) vr[b][v] = u32x4{0u, 0u, 0u, 0u};
    }
    // V key pairs (v = 0,1) and (v = 2,3): element e of this lane's d-chunk
    uint32_t vp[2][2][8];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const u32x4 A = vr[b][2 * pr];
        const u32x4 B = vr[b][2 * pr + 1];
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
          vp[b][pr][2 * dw] = __builtin_amdgcn_perm(B[dw], A[dw], 0x05040100u);
          vp[b][pr][2 * dw + 1] = __builtin_amdgcn_perm(B[dw], A[dw], 0x07060302u);
        }
      }
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const u32x4 ph = p_lds[wave][grp][h];
      if (any_upd) {
        const float al = x_lds[wave][grp][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = acc[h][e];
        t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ph[0]), as_bf16x2(vp[0][0][e]), t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ph[1]), as_bf16x2(vp[0][1][e]), t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ph[2]), as_bf16x2(vp[1][0][e]), t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ph[3]), as_bf16x2(vp[1][1][e]), t, false);
        acc[h][e] = t;
      }
    }
  }

  // merge the four lane groups of this wavefront
  float M = m;
  M = fmaxf(M, shfl_xor(M, 16));
  M = fmaxf(M, shfl_xor(M, 32));
  const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
  float L = lsum * f;
  L += shfl_xor(L, 16);
  L += shfl_xor(L, 32);
  x_lds[wave][grp][lo] = f;
  if (grp == 0) l_lds[wave][lo] = L;
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    const float fh = x_lds[wave][grp][h];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = acc[h][e] * fh;
      t += shfl_xor(t, 16);
      t += shfl_xor(t, 32);
      acc[h][e] = t;
    }
  }

  if (nsplit == 1) {  // the whole request in one item: normalise and write
    if (active && grp == 0) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        if (h < G) {
          const float Lh = l_lds[wave][h];
          const float inv = Lh > 0.f ? 1.f / Lh : 0.f;
          uint4 out;
          out.x = pack_bf16x2(acc[h][0] * inv, acc[h][1] * inv);
          out.y = pack_bf16x2(acc[h][2] * inv, acc[h][3] * inv);
          out.z = pack_bf16x2(acc[h][4] * inv, acc[h][5] * inv);
          out.w = pack_bf16x2(acc[h][6] * inv, acc[h][7] * inv);
          *reinterpret_cast<uint4*>(a.o + ((tok * a.Hq) + (int64_t)g * G + h) * kHeadDim + lo * 8) = out;
        }
      }
    }
    return;
  }

  // several items: publish this item's (acc, max, sum) for the merge launch
  if (active && grp == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (h < G) {
        float* dst = a.ws_acc + (((int64_t)item * a.Hq) + (int64_t)g * G + h) * kHeadDim + lo * 8;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      }
    }
    if (lo < G) {
      float* ml = a.ws_ml + (((int64_t)item * a.Hq) + (int64_t)g * G + lo) * 2;
      ml[0] = M;
      ml[1] = L;
    }
  }
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
  int gp = 1;
  while (gp < a.group) gp <<= 1;
  switch (gp) {
    case 1:
    case 2:
    case 4: hipLaunchKernelGGL(decode_kernel<4>, grid, dim3(64 * kWaves), 0, s, a); break;
    case 8: hipLaunchKernelGGL(decode_kernel<8>, grid, dim3(64 * kWaves), 0, s, a); break;
    default: hipLaunchKernelGGL(decode_kernel<16>, grid, dim3(64 * kWaves), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)a.num_decode, (unsigned)((a.Hq + 1) / 2)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
