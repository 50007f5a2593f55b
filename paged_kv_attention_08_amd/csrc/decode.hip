// paged_decode_attn: split-K ("flash-decoding") attention of one new token per
// request over K/V rows gathered through the page table.
//
// mini-sglang learning notes, kernel passage: decode is memory bound, its cost
// is the gather of variable-length K/V, and it is parallelised across the KV
// sequence.  Deep dive 5.2: online softmax keeps a running max and sum so no
// score vector is stored.
//
// Work decomposition (from the plan written by build_attn_metadata): the
// decode work is the flat sequence of (request, group of HG KV heads, 32-key
// tile), request by request, each (request, group) "segment" holding
// ceil(device_len / 32) tiles; HG is the largest of 8, 4, 2, 1 dividing Hkv.
// A fixed set of kDecodeWaves / HG "runs" of HG wavefronts each (8 wavefronts
// per workgroup, one workgroup per CU, all resident at once) take equal shares
// of `per` consecutive tiles, so every run has the same work whatever the mix
// of lengths (a per-request split into items of a fixed size left a quarter
// of the wavefront slots idle on average at the serving-decode batch).  The
// wavefronts of a run walk the same tiles, one KV head of the group each, so
// at any time they read adjacent heads (2 KiB contiguous at HG = 8: whole K
// and V rows of an 8-KV-head pool, measured 7% faster than 1 KiB pieces on
// the serving-decode batch) of the same pool rows.  A wavefront walks its run
// tile by tile across segment boundaries, keeping its loads in flight across
// them; a segment that lies wholly inside the run is normalised and written
// directly, and the piece of a segment shared with a neighbouring run is
// published as a partial state.
//
// Per tile and wavefront (lane = 16 * grp + lo):
//   * lanes 0..31 read the 32 page-table entries (requested two tiles ahead,
//     possibly of the next segment);
//     rows are broadcast with lane shuffles.  Each 16-lane group then loads
//     one whole 256-byte head row of K and of V per instruction (4 rows per
//     instruction, 8 + 8 loads per lane).  A missing key (past device_len)
//     loads nothing and is masked: every key of a tile of a one-key padding
//     request used to read pool row 0, and those loads piled onto one row.
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
// segment inside one run is written directly; otherwise each run publishes its
// piece's (acc, max, sum) to the workspace (slot 0: the piece of the segment
// the run started inside, slot 1: the one it ends inside) and a second launch
// rescales the pieces of each (request, query head) to their common max in one
// pass.
// (Merging inside the first launch would need device-scope fences, which on
// this chip write back and invalidate a whole L2 per workgroup; the launch
// boundary orders the two kernels for free.)
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kTileKeys = kDecodeTileKeys;
constexpr int kWaves = kDecodeWgWaves;  // wavefronts per workgroup: 8 / HG runs (no barrier between them)
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

// Uniform reads of data no launch of this call writes (plan, lengths, token
// offsets, table rows) go through the constant address space, so they become
// scalar loads with their own counter: as vector loads, every wait for them
// also waited for the 16 row loads just issued for the next tile.  (Measured
// neutral at the serving, long-context and page-64 batches: the other
// wavefront of each SIMD covered that stall; the loop now keeps a tile of rows
// in flight per wavefront as intended.)
template <typename T>
__device__ inline T ldu(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Position in the flat decode order (uniform across the wavefront).
struct Cursor {
  int32_t i;    // request
  int32_t g;    // group of KV heads
  int32_t kti;  // tile within the segment
  int32_t n;    // tiles per segment of request i
  int32_t seg;  // flat index of the segment's first tile
  int32_t dl;   // device_len of request i
};

__global__ void __launch_bounds__(64 * kWaves, 1) decode_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[kWaves][kTileKeys * kKsPitch];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kWaves][kTileKeys * kVsPitch];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15;
  const int grp = lane >> 4;
  const int32_t* header = reinterpret_cast<const int32_t*>(a.plan);
  const int32_t total = ldu(header);
  const int32_t per = ldu(header + 1);
  const int Hkv = a.Hkv;
  const int HG = decode_heads_per_group(Hkv);
  const int Hg = Hkv / HG;
  const int hw = wave % HG;  // this wavefront's KV head within the group
  const int32_t run = blockIdx.x * (kWaves / HG) + wave / HG;
  const int64_t f0l = (int64_t)run * per;
  if (f0l >= total) return;  // uniform for the run; no workgroup barrier below
  const int32_t f0 = (int32_t)f0l;
  const int32_t f1 = (int32_t)min<int64_t>(f0l + per, total);
  const int32_t* tptr = reinterpret_cast<const int32_t*>(a.plan + a.layout.dec_tiles_off);
  const int G = a.group;

  // the request holding flat tile f0: Hg * tptr[i] <= f0 < Hg * tptr[i + 1]
  Cursor cc;
  {
    int lo_i = 0, hi_i = a.num_decode;  // tptr[num_decode] * Hg = total > f0
    while (hi_i - lo_i > 1) {
      const int mid = (lo_i + hi_i) >> 1;
      if ((int64_t)Hg * ldu(tptr + mid) <= f0) lo_i = mid;
      else hi_i = mid;
    }
    cc.i = lo_i;
    const int32_t t_lo = ldu(tptr + lo_i);
    cc.n = ldu(tptr + lo_i + 1) - t_lo;
    const int32_t local = f0 - Hg * t_lo;
    cc.g = local / cc.n;
    cc.kti = local - cc.g * cc.n;
    cc.seg = Hg * t_lo + cc.g * cc.n;
    cc.dl = ldu(a.device_len + lo_i);
  }
  // next tile of the flat order (only called while one exists in the run)
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    if (++c.kti == c.n) {
      c.kti = 0;
      c.seg += c.n;
      if (++c.g == Hg) {
        c.g = 0;
        do {
          ++c.i;
        } while (ldu(tptr + c.i + 1) == ldu(tptr + c.i));  // requests without decode tiles
        c.n = ldu(tptr + c.i + 1) - ldu(tptr + c.i);
        c.dl = ldu(a.device_len + c.i);
      }
    }
  };
  auto token_of = [&](const Cursor& c) -> int64_t { return ldu(a.qo_indptr + c.i); };
  // this wavefront's KV head in c's group
  auto head_of = [&](const Cursor& c) -> int { return c.g * HG + hw; };

  uint16_t* ktile = ks[wave];
  uint16_t* vtile = vs[wave];
  const int64_t stride = a.row_stride;

  // B operand of S^T: the G query heads of KV head g (zero for padded columns)
  auto load_q = [&](const Cursor& c, bf16x8 (&qo)[4]) __attribute__((always_inline)) {
    const int64_t tok = token_of(c);
    const int h = head_of(c);
    const bool ok = tok >= 0 && tok < a.T && lo < G;
    const uint16_t* qrow = a.q + ((ok ? tok : 0) * a.Hq + (ok ? (int64_t)h * G + lo : 0)) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = load16(qrow + (grp * 4 + kk) * 8);
      qo[kk] = as_bf16x8(v);
    }
  };
  // Page-table entries of the 32 keys of c's tile: every lane loads (lanes
  // 32..63 and keys past device_len re-read an in-range entry).
  auto load_entries = [&](const Cursor& c) -> int32_t {
    const int32_t* pt_row = a.page_table + (int64_t)ldu(a.table_idx + c.i) * a.W;
    return pt_row[min(c.kti * kTileKeys + (lane & 31), c.dl - 1)];
  };
  // -1 marks a key past device_len or an entry outside the pool (reported)
  auto check_entries = [&](const Cursor& c, int32_t e) -> int32_t {
    const bool in_range = lane < kTileKeys && c.kti * kTileKeys + lane < c.dl;
    if (in_range && (e < 0 || (int64_t)e >= a.num_pool_rows)) {
      raise_status(a.status, PKV_STATUS_BAD_PAGE_ROW);
      e = -1;
    }
    return in_range ? e : -1;
  };
  u32x4 kr[8], vr[8];  // the rows of the tile in flight
  auto issue = [&](const Cursor& c, int32_t e) __attribute__((always_inline)) {
    // loader: load u (0..7) of lane l moves 16 bytes (dims 8 (l % 16) ..) of
    // key 4 u + l / 16: each 16-lane group reads one whole 256-byte head row
    const int h = head_of(c);
    const uint16_t* kbase = a.k_pool + (int64_t)h * kHeadDim + lo * 8;
    const uint16_t* vbase = a.v_pool + (int64_t)h * kHeadDim + lo * 8;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int32_t row = __shfl(e, 4 * u + (lane >> 4), 64);
      kr[u] = u32x4{0u, 0u, 0u, 0u};
      vr[u] = u32x4{0u, 0u, 0u, 0u};
      if (row >= 0) {  // the same for the 16 lanes of a group
        kr[u] = load16_stream(kbase + (int64_t)row * stride);
        vr[u] = load16_stream(vbase + (int64_t)row * stride);
      }
    }
  };

  const float c = a.scale_log2;
  float m = -INFINITY;  // running max of head lo, in log2 units (same in all four lane groups)
  float lsum = 0.f;     // this lane group's part of the running sum
  f32x4 oacc[8];        // O^T block mb: dims 16 mb + 4 grp + v of head lo
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) oacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: rows of tile f0 in flight, entries of tile f0 + 1 requested, q of f0's segment
  Cursor cl = cc;  // the tile whose rows are in flight
  Cursor ce = cc;  // the tile whose entries are in flight
  int32_t ent = check_entries(ce, load_entries(ce));
  issue(cl, ent);
  uint32_t valid_next = (uint32_t)__ballot(ent >= 0);  // bit k: key k of the tile has a row
  int32_t ent_raw = -1;
  if (f0 + 1 < f1) {
    advance(ce);
    ent_raw = load_entries(ce);
  }
  bf16x8 qop[4], qnext[4];
  load_q(cc, qop);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qnext[kk] = qop[kk];

  for (int32_t f = f0; f < f1; ++f) {
    const uint32_t valid = valid_next;
    // this tile's rows -> the wavefront's row-major LDS tiles (a missing key's rows are zero)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = 4 * u + (lane >> 4);
      *reinterpret_cast<u32x4*>(&ktile[key * kKsPitch + lo * 8]) = kr[u];
      *reinterpret_cast<u32x4*>(&vtile[key * kVsPitch + lo * 8]) = vr[u];
    }
    // the next tile's rows (possibly of the next segment) go out now and stay
    // in flight while this one is computed
    if (f + 1 < f1) {
      advance(cl);
      ent = check_entries(cl, ent_raw);
      issue(cl, ent);
      valid_next = (uint32_t)__ballot(ent >= 0);
      if (cl.kti == 0) load_q(cl, qnext);  // a new segment starts with the next tile
      if (f + 2 < f1) {
        advance(ce);
        ent_raw = load_entries(ce);
      }
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

    // end of the segment or of the run: finish this piece
    const bool seg_end = cc.kti == cc.n - 1;
    if (seg_end || f + 1 == f1) {
      // the four lane groups share the max: only the sums need reducing
      float L = lsum;
      L += shfl_xor(L, 16);
      L += shfl_xor(L, 32);
      const int64_t tok = token_of(cc);
      const bool tok_ok = tok >= 0 && tok < a.T;
      if (!tok_ok && lane == 0) raise_status(a.status, PKV_STATUS_TOKEN_COUNT);
      const bool started_before = cc.seg < f0;
      const int h = head_of(cc);
      if (tok_ok && lo < G) {
        const int64_t hq = (int64_t)h * G + lo;
        if (!started_before && seg_end) {  // the whole segment: normalise and write
          const float inv = L > 0.f ? 1.f / L : 0.f;
          uint16_t* orow = a.o + (tok * a.Hq + hq) * kHeadDim + 4 * grp;
#pragma unroll
          for (int mb = 0; mb < 8; ++mb)
            *reinterpret_cast<uint2*>(orow + 16 * mb) = make_uint2(pack_bf16x2(oacc[mb][0] * inv, oacc[mb][1] * inv),
                                                                  pack_bf16x2(oacc[mb][2] * inv, oacc[mb][3] * inv));
        } else {  // a piece of a shared segment: publish (acc, max, sum)
          const int64_t slot = (((int64_t)run * 2 + (started_before ? 0 : 1)) * HG + hw) * G + lo;
          float* dst = a.ws_acc + slot * kHeadDim + 4 * grp;
#pragma unroll
          for (int mb = 0; mb < 8; ++mb)
            *reinterpret_cast<float4*>(dst + 16 * mb) = make_float4(oacc[mb][0], oacc[mb][1], oacc[mb][2], oacc[mb][3]);
          if (grp == 0) *reinterpret_cast<float2*>(a.ws_ml + slot * 2) = make_float2(m, L);
        }
      }
      m = -INFINITY;
      lsum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) oacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qop[kk] = qnext[kk];
    }
    if (f + 1 < f1) advance(cc);
  }
}

// One workgroup per (request, pair of query heads), one thread per dimension:
// the pieces of a segment shared by runs w0 .. w1 are run w0's slot 1 and
// slot 0 of runs w0 + 1 .. w1 (each at the KV head's wavefront); a single
// pass with a running max combines them (their loads do not depend on the
// running state, so they overlap).
__global__ void __launch_bounds__(256) decode_merge_kernel(AttnArgs a) {
  const int i = blockIdx.x;
  const int hq = blockIdx.y * 2 + (threadIdx.x >> 7);
  const int d = threadIdx.x & 127;
  if (hq >= a.Hq) return;
  const int32_t* header = reinterpret_cast<const int32_t*>(a.plan);
  const int32_t per = header[1];
  const int32_t* tptr = reinterpret_cast<const int32_t*>(a.plan + a.layout.dec_tiles_off);
  const int32_t n = tptr[i + 1] - tptr[i];
  if (n == 0) return;  // not a valid decode request
  const int G = a.group;
  const int g = hq / G;
  const int gh = hq - g * G;
  const int HG = decode_heads_per_group(a.Hkv);
  const int gg = g / HG;
  const int wv = g - gg * HG;
  const int64_t seg = (int64_t)(a.Hkv / HG) * tptr[i] + (int64_t)gg * n;
  const int64_t w0 = seg / per;
  const int64_t w1 = (seg + n - 1) / per;
  if (w0 == w1) return;  // written by the first launch
  const int64_t tok = a.qo_indptr[i];
  if (tok < 0 || tok >= a.T) return;
  float Mx = -INFINITY, den = 0.f, num = 0.f;
#pragma unroll 4
  for (int64_t w = w0; w <= w1; ++w) {
    const int64_t slot = ((w * 2 + (w == w0 ? 1 : 0)) * HG + wv) * G + gh;
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + slot * 2);
    const float aj = a.ws_acc[slot * kHeadDim + d];
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
  hipLaunchKernelGGL(decode_kernel, dim3(kDecodeWaves / kWaves), dim3(64 * kWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)a.num_decode, (unsigned)((a.Hq + 1) / 2)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
