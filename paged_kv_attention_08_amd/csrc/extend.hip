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
//   * the workgroup gathers 64 K rows and 64 V rows of head g straight into
//     LDS (global_load_lds_dwordx4: the data never passes through registers)
//     three tiles ahead, into four LDS stages (tile n in stage n % 4):
//     wavefront w takes keys 8w..8w+7, each 16-lane group one whole 256-byte
//     head row per load (16 bytes per lane), so a load instruction fills 4
//     rows, 1 KB contiguous in LDS.  (With one key per lane, every
//     instruction touched 64 scattered rows and half the address
//     translations missed the per-CU TLB.)  Rows are unpadded; their 16-byte
//     chunks are permuted (a XOR swizzle chosen when the row is gathered) so
//     that the operand reads below hit distinct LDS banks.  The page-table
//     entries travel the same way, into a small per-wavefront ring, six tiles
//     ahead.  These loads and every wait for them are written out by hand
//     (the compiler would wait for all of them before any LDS read); one
//     barrier per tile;
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
constexpr int kWaves = 8;
static_assert(kExtendRows == 32 * kWaves, "one 32-row block per wavefront");
constexpr int kWaveKeys = kKeyTile / kWaves;  // keys of a tile one wavefront gathers
constexpr int kLoads = kWaveKeys / 4;         // 16-byte loads per lane per tile and per K / V (4 rows per load)
static_assert(kLoads == 2, "two 4-row loads per wavefront and operand");
constexpr int kStages = 4;                                       // LDS stages: tile n in stage n % 4
constexpr int kTileBytes = kKeyTile * kHeadDim * 2;              // 16 KB, unpadded rows
constexpr int kVRegion = kStages * kTileBytes;                   // V tiles after the K tiles
constexpr int kRingOff = 2 * kVRegion;                           // page-table entry ring
constexpr int kRingSlots = 4;
constexpr int kRingWave = 256;                                   // bytes per wavefront and slot
constexpr int kLdsBytes = kRingOff + kRingSlots * kWaves * kRingWave;
static_assert(kLdsBytes <= 160 * 1024, "fits the CU's LDS");
// Every K operand read (stage, 32-key block) and V operand read (stage,
// block, 16-key half) is a 16-bit immediate offset from a per-lane base: the
// K stages fill the first 64 KB and the V stages the next.
static_assert((kStages - 1) * kTileBytes + 8192 < 65536, "K read offsets fit the immediate field");
// Load schedule, per iteration n (tile n): the entries of tile n + kEntryLead,
// the rows of tile n + kRowLead (from entries read into registers during
// iteration n - 1).  Exactly kOpsPerTile vector-memory instructions per
// iteration and wavefront.
constexpr int kRowOps = 2 * kLoads;                 // K and V row loads per iteration
constexpr int kOpsPerTile = 1 + kRowOps;            // + one entry load
constexpr int kRowLead = kStages - 1;               // rows of tile n + 3
constexpr int kEntryLead = kRowLead + 3;            // entries of tile n + 6
static_assert(kEntryLead - kRowLead < kRingSlots, "ring slots outlive their reads");
// Rows of tile n + 1 (issued in iteration n - 2) are followed by two whole
// iterations' ops when iteration n ends.
constexpr int kWaitRows = 2 * kOpsPerTile;
// Entries of tile n + 4 (issued first in iteration n - 2) are followed by the
// row loads of iteration n - 2 and two whole iterations when iteration n has
// issued its rows.
constexpr int kWaitEntries = kRowOps + 2 * kOpsPerTile;

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ inline float dot2_bf16(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w), __builtin_bit_cast(bf16x2v, 0x3F803F80u), acc, false);
}

// Swizzle of a tile row's 16 16-byte chunks: logical chunk c of row r sits in
// slot c ^ swz(r).  Any 16 consecutive rows map one logical chunk to 16
// distinct slots (the K operand reads: 16 lanes, 16 rows, one chunk), and any
// 4 rows 4-aligned put chunks 4b..4b+3 in 16 distinct slots (the transpose
// reads of V: 4 rows x 4 chunks per 32 lanes), so neither read conflicts.
__device__ inline int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Loads that write LDS directly (the data never passes through registers).
// They are issued as inline assembly so that the compiler, which would
// otherwise wait for every such load before any LDS read, leaves them in
// flight; every wait for them below is explicit.  Lane l's bytes land at LDS
// byte address m0 + size * l.  One wait state is needed between the write of
// m0 and its read by the load.
__device__ inline void lds_load16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(g) : "memory", "m0");
}
__device__ inline void lds_load4(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_addr), "v"(g) : "memory", "m0");
}

__global__ void __launch_bounds__(64 * kWaves, 8 / kWaves) extend_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];

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

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  const int n_kt = (kv_end + kKeyTile - 1) / kKeyTile;  // key tiles of the item
  const int32_t* pt_row = a.page_table + (int64_t)a.table_idx[i] * a.W;
  const uint32_t row_elems = (uint32_t)a.row_stride;  // < 2^31, checked on the host
  const uint32_t n_rows = (uint32_t)a.num_pool_rows;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // Gather of tile n (keys 64 n ..): load u (0, 1) of lane l in wavefront w
  // moves the 16-byte chunk that belongs in slot l % 16 of tile row
  // 8 w + 4 u + l / 16, i.e. logical chunk (l % 16) ^ swz(row), so one
  // instruction fills 4 whole rows (1 KB, contiguous in LDS).  Keys past
  // kv_end re-read the last valid key's row: finite data, only in the last
  // tile, which is always masked, so their probabilities are exactly 0; tiles
  // past the end are gathered the same way, so every tile issues the same
  // loads and the explicit wait counts hold on every path.
  const uint16_t* kbase = a.k_pool + (int64_t)g * kHeadDim;
  const uint16_t* vbase = a.v_pool + (int64_t)g * kHeadDim;
  uint32_t chunk_el[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) chunk_el[u] = (uint32_t)(((lane & 15) ^ swz(4 * u + (lane >> 4))) * 8);
  // (8 w + 4 u + l / 16) & 15 = 4 u + l / 16 + 8 (w & 1); swz depends on the
  // row's low 4 bits, and 8 (w & 1) only sets bit 3
  if (wave & 1) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) chunk_el[u] = (uint32_t)(((lane & 15) ^ swz(8 + 4 * u + (lane >> 4))) * 8);
  }

  // Page-table entries of tile n (keys 8 w .. 8 w + 7 of each wavefront) go
  // to ring slot n % 4 of the wavefront: lane l loads key 8 w + l % 8 (the
  // eight copies are harmless), lane l later reads keys 8 w + 4 u + l / 16.
  // A slot is written in iteration n - 6 and read in iteration n - 4; the
  // next write to it comes in iteration n - 2.
  const uint32_t ring = lds_base + kRingOff + wave * kRingWave;
  auto load_entries = [&](int n) __attribute__((always_inline)) {
    const int key = min(n * kKeyTile + kWaveKeys * wave + (lane & 7), kv_end - 1);
    lds_load4(pt_row + key, ring + (uint32_t)((n & (kRingSlots - 1)) * kWaves * kRingWave));
  };
  // Issue step of iteration n: the entries of tile n + 6, then the K/V rows of
  // tile n + 3 (into the stage of tile n - 1, which every wavefront finished
  // before the last barrier) from the entries read into registers during the
  // previous iteration, then, for the next iteration, the entries of tile
  // n + 4 from the ring.  A status atomic on a bad row only adds
  // vector-memory ops, which makes every count-based wait stricter.
  uint32_t ent[kLoads];
  auto read_entries = [&](int m) __attribute__((always_inline)) {
    const uint32_t slot = (uint32_t)kRingOff + wave * kRingWave + (uint32_t)((m & (kRingSlots - 1)) * kWaves * kRingWave);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) ent[u] = *reinterpret_cast<const uint32_t*>(lds + slot + 4 * (4 * u + (lane >> 4)));
  };
  auto issue = [&](int n) __attribute__((always_inline)) {
    load_entries(n + kEntryLead);
    const int m = n + kRowLead;
    uint32_t r[kLoads];
    bool bad = false;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      r[u] = ent[u];
      const bool b = r[u] >= n_rows;  // also catches negative entries
      bad |= b;
      r[u] = b ? 0u : r[u];
    }
    const uint32_t stage_k = lds_base + (uint32_t)((m & (kStages - 1)) * kTileBytes);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const uint64_t off = (uint64_t)r[u] * row_elems + chunk_el[u];
      const uint32_t dst = stage_k + (uint32_t)((kWaveKeys * wave + 4 * u) * kHeadDim * 2);
      lds_load16(kbase + off, dst);
      lds_load16(vbase + off, dst + kVRegion);
    }
    if (bad) raise_status(a.status, PKV_STATUS_BAD_PAGE_ROW);
    // everything older than those entries is tile n's rows, needed already
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitEntries) : "memory");
    read_entries(n + kRowLead + 1);
  };
  // End of a tile: this wavefront's rows of the next tile are in LDS and
  // every LDS read of the current tile has returned; after the barrier every
  // wavefront's rows are.
  auto finish = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kWaitRows) : "memory");
  };

  // per-lane LDS read addresses (bytes from the stage's K or V tile)
  // K operand: row 32 mb + l32, logical chunk half + 2 jj ->
  //   slot (2 jj) ^ (half ^ swz(l32 & 15)); row offset l32 * 256 + mb * 8192
  uint32_t kaddr[8];
  {
    const int hk = half ^ swz(l32 & 15);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) kaddr[jj] = (uint32_t)(l32 * 256 + (((2 * jj) ^ hk) << 4));
  }
  // V^T operand (transpose reads): in each 16-lane group lane j16 reads row
  // key0 + j16 / 4 (and 8 rows on), logical elements nb * 32 + 16 ((l / 16) & 1)
  // + 4 (j16 & 3); the XOR with 64 nb moves chunk 4 nb + b to its slot
  uint32_t vaddr[2][4];
  {
    const int j16 = lane & 15;
    const int b = ((lane >> 4) & 1) * 2 + ((j16 & 3) >> 1);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 4 * half + (j16 >> 2) + 8 * p;
      const int base = r * 256 + ((b ^ swz(r)) << 4) + 8 * (j16 & 1);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) vaddr[p][nb] = (uint32_t)(kVRegion + (base ^ (64 * nb)));
    }
  }

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

  // One 64-key tile n in stage S.  MASK: the tile reaches past the first
  // row's position, so keys beyond a row's own position are masked (diagonal
  // and ragged end).
  auto key_tile = [&](int n, auto stage_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    const int kt = n * kKeyTile;
    const bool MASK = kt >= kt_mask;  // uniform
    const uint8_t* ks = lds + S * kTileBytes;
    const uint8_t* vs = lds + S * kTileBytes;  // vaddr holds the V region offset

    // S^T = K Q^T : two 32-key blocks (raw scores, scale folded into exp below);
    // the two accumulation chains alternate and the K operands are read from
    // LDS four MFMAs ahead, the first four before the next tiles' loads are
    // issued.  sched_barrier pins that order.
    f32x16 sacc[2];
    auto kread = [&](int j) __attribute__((always_inline)) {
      return as_bf16x8(*reinterpret_cast<const uint4*>(ks + kaddr[j >> 1] + (j & 1) * 8192));
    };
    bf16x8 kb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j] = kread(j);
    __builtin_amdgcn_sched_barrier(0);
    issue(n);
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
      // key kt + 4 half + k_off > pos  <=>  k_off > pos - kt - 4 half: one
      // subtraction per lane, then a compare against a constant per element
      const int lim = pos - kt - 4 * half;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * mb + 8 * (v >> 2) + (v & 3) > lim) sacc[mb][v] = -INFINITY;
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
      const int roff = mb * 8192 + kq * 4096;
      const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(vs + vaddr[0][nb] + roff));
      const v4s r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(vs + vaddr[1][nb] + roff));
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
      // the first tile of an item (every row's m was -inf) has nothing to rescale
      if (__ballot(alpha != 0.f) != 0) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[nb][v] *= alpha;
      }
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
    finish();
  };

  // Prologue: the entries of tiles 0 .. 2, waited for together with the q
  // rows (the empty asm statements use q here, so that the compiler's own
  // wait for the q loads comes before the loop and not inside it), tile 0's
  // entries into registers, then the issue steps of iterations -3 .. -1 (rows
  // of tiles 0 .. 2); after the first barrier tile 0's rows are in LDS.
  load_entries(0);
  load_entries(1);
  load_entries(2);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) asm volatile("" ::"v"(qop[kk]));
  read_entries(0);
  issue(-3);
  issue(-2);
  issue(-1);
  finish();
  int n = 0;
  for (; n + kStages <= n_kt; n += kStages) {
    key_tile(n, std::integral_constant<int, 0>{});
    key_tile(n + 1, std::integral_constant<int, 1>{});
    key_tile(n + 2, std::integral_constant<int, 2>{});
    key_tile(n + 3, std::integral_constant<int, 3>{});
  }
  if (n < n_kt) key_tile(n, std::integral_constant<int, 0>{});
  if (n + 1 < n_kt) key_tile(n + 1, std::integral_constant<int, 1>{});
  if (n + 2 < n_kt) key_tile(n + 2, std::integral_constant<int, 2>{});
  // no load may still be writing LDS when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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
