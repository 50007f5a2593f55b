// build_attn_metadata: page-table write for the batch's new tokens, out_loc,
// positions, running totals and the attention plan.
//
// mini-sglang learning notes, page-table passage: the scheduler counts, page
// aligned, the new pages each request needs for [cached_len, device_len),
// takes them from free_slots and writes the page table with raw physical
// positions; the Batch then carries positions and out_loc.  "SGLang source
// guide", main line 3: the same quantities are seq_lens, extend_prefix_lens,
// extend_seq_lens, req_pool_indices and out_cache_loc.
//
// One launch on the caller's stream, plan_kernel:
//   workgroup 0: per-request validation, running totals (qo_indptr,
//                kv_indptr, last_indices, alloc offsets), the decode tile
//                offsets and per-run share (the decode kernel splits the flat
//                sequence of (request, group of KV heads, key tile) evenly
//                over its runs) and the extend tile list, ordered by key
//                count, most first (so the last workgroups to start are the
//                shortest and the CUs finish together);
//   workgroups 1.. (map blocks, kMapTokens new tokens each): rebuild the two
//                running totals they need in LDS, find each token's request
//                by binary search and write page_table, out_loc and
//                positions; with K/V given (build_attn_metadata_store) they
//                also copy the tokens' K/V rows into the pool.
// A batch of more than kFuseReqs requests (too many for the LDS copy of the
// running totals) maps its tokens in a second launch instead, token_kernel
// (one thread per new token, binary search over qo_indptr in memory), and is
// stored by kv_store after it.
// Inside a replayed decode graph the batch is padded here too (learning notes
// graph passage: padding requests fill the batch up to the captured size and
// point at the dummy page): requests from pad_from on are taken as dummy
// requests whatever the arrays hold, and plan_kernel writes their values into
// the arrays for the kernels that follow.
// Integer work only; results are bit-exact by construction.
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kScanVals = 5;
constexpr int kSortBuckets = 1024;  // extend tiles sorted by key count in steps of 64 keys (capped)
constexpr int kFuseReqs = 1024;     // most requests whose running totals a map block copies to LDS
constexpr int kMapTokens = 8;       // new tokens per map block
constexpr int kCopyVec = 4;         // 16-byte K (and V) vectors a map-block thread loads before storing
static_assert(kSortBuckets % kPlanThreads == 0, "whole buckets per thread");

struct ReqInfo {
  bool valid;
  int32_t ext, dl, new_pages, dtiles, tiles;
};

// (table row, cached_len, device_len) of request i: a padding request from
// pad_from on is a dummy request on the all-zero table row.
struct ReqFields {
  int32_t r, c, dl;
};

__device__ inline ReqFields req_fields(const MetaArgs& a, int i) {
  if (i >= a.pad_from) return {a.dummy_row, 0, 1};
  return {a.table_idx[i], a.cached_len[i], a.device_len[i]};
}

__device__ inline int32_t ceil_div_pow2(int32_t x, int32_t shift) {
  return (x + (1 << shift) - 1) >> shift;
}

__device__ inline bool request_ok(const MetaArgs& a, int i, const ReqFields& f, int32_t* bits) {
  const int32_t r = f.r;
  const int32_t c = f.c;
  const int32_t dl = f.dl;
  bool ok = true;
  if (r < 0 || r >= a.R) { *bits |= PKV_STATUS_BAD_TABLE_IDX; ok = false; }
  if (c < 0 || c > dl || dl > a.W) { *bits |= PKV_STATUS_BAD_LENGTHS; ok = false; }
  if (i < a.num_decode && dl - c != 1) { *bits |= PKV_STATUS_BAD_DECODE; ok = false; }
  return ok;
}

// Exclusive scan of kScanVals ints over the whole workgroup; returns totals.
__device__ inline void block_scan(int32_t (&v)[kScanVals], int32_t (&excl)[kScanVals],
                                  int32_t (&tot)[kScanVals], int32_t (*smem)[kPlanWaves]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int32_t inc[kScanVals];
#pragma unroll
  for (int q = 0; q < kScanVals; ++q) {
    int32_t x = v[q];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    inc[q] = x;
    if (lane == 63) smem[q][wave] = x;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kScanVals; ++q) {
    int32_t before = 0, all = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      const int32_t s = smem[q][w];
      if (w < wave) before += s;
      all += s;
    }
    excl[q] = before + inc[q] - v[q];
    tot[q] = all;
  }
  __syncthreads();
}

// New tokens and new pages of request i (the running totals' terms; invalid
// lengths count no pages, as the allocator gives them none).
__device__ inline void req_counts(const MetaArgs& a, const ReqFields& f, int32_t* ext, int32_t* new_pages) {
  const int32_t c = f.c, dl = f.dl, s = a.page_shift;
  *ext = dl > c && c >= 0 ? dl - c : 0;
  *new_pages = (c >= 0 && c <= dl) ? ceil_div_pow2(dl, s) - ceil_div_pow2(c, s) : 0;
}

// Token t of the batch: its request i (qo[i] <= t < qo[i + 1], by binary
// search over qo, the running totals in global memory or LDS), its logical
// position j, and its row in the request's partial page or new pages.  row is
// -1 for a token that gets no row; bits holds the status bits a bad
// page-table entry or alloc entry raises (an invalid request was already
// reported by plan_kernel).
struct TokenRow {
  int32_t row, j, table_row, bits;
};

__device__ inline TokenRow token_row(const MetaArgs& a, int64_t t, const int32_t* qo, const int32_t* alloc_ptr) {
  TokenRow out = {-1, -1, -1, 0};
  if (t >= qo[a.B]) return out;  // fewer new tokens than num_tokens (flagged by plan_kernel)
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qo[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int i = lo;
  int32_t bits = 0;
  const ReqFields f = req_fields(a, i);
  if (!request_ok(a, i, f, &bits)) return out;
  const int32_t c = f.c;
  const int32_t j = c + (int32_t)(t - qo[i]);
  const int32_t s = a.page_shift;
  const int32_t slot = j & ((1 << s) - 1);
  const int32_t first_new_page = ceil_div_pow2(c, s);
  const int32_t lp = j >> s;
  int64_t row;
  if (lp < first_new_page) {
    // the request's partially filled last cached page (an entry before cached_len)
    row = (int64_t)a.page_table[(int64_t)f.r * a.W + (j - slot)] + slot;
    if (row < 0 || row >= a.num_pool_rows) bits |= PKV_STATUS_BAD_PAGE_ROW;
  } else if (i >= a.pad_from) {
    row = slot;  // a padding request's one new row: the dummy page
  } else {
    const int64_t ai = (int64_t)alloc_ptr[i] + (lp - first_new_page);
    if (ai >= a.num_alloc) {
      bits |= PKV_STATUS_BAD_ALLOC;
      row = -1;
    } else {
      const int32_t pr = a.alloc_rows[ai];
      row = (int64_t)pr + slot;
      if (pr < 0 || (pr & ((1 << s) - 1)) != 0 || row >= a.num_pool_rows) bits |= PKV_STATUS_BAD_ALLOC;
    }
  }
  out.bits = bits;
  if (!bits) {
    out.row = (int32_t)row;
    out.j = j;
    out.table_row = f.r;
  }
  return out;
}

// Writes page_table, out_loc and positions of token t and returns its row.  A
// token that gets no row is marked -1 in out_loc and positions, so the store
// and RoPE calls skip it instead of reusing a stale row.
__device__ inline int32_t map_token(const MetaArgs& a, int64_t t, const int32_t* qo, const int32_t* alloc_ptr) {
  const TokenRow tr = token_row(a, t, qo, alloc_ptr);
  if (tr.bits) raise_status(a.status, tr.bits);
  if (tr.row < 0) {
    a.out_loc[t] = -1;
    a.positions[t] = -1;
    return -1;
  }
  a.page_table[(int64_t)tr.table_row * a.W + tr.j] = tr.row;
  a.out_loc[t] = tr.row;
  a.positions[t] = tr.j;
  return tr.row;
}

// A map block (workgroups 1.. of plan_kernel): it rebuilds the two running
// totals it needs (new tokens and new pages per request) in LDS, maps its
// kMapTokens tokens as map_token does and, when K/V are given, copies their K
// and V rows into the pool, consecutive threads on consecutive 16-byte
// vectors of a row, each thread loading up to kCopyVec vectors of each before
// storing them.  Workgroup 0 writes the plan meanwhile; the mapping reads only
// page-table entries before each request's cached_len, which no workgroup of
// the launch writes.
__device__ inline void map_block(const MetaArgs& a, int32_t* s_qo, int32_t* s_ap, int32_t (*smem)[kPlanWaves],
                                 int32_t* s_rows) {
  const int tid = threadIdx.x;
  int32_t carry_q = 0, carry_a = 0;
  if (tid == 0) {
    s_qo[0] = 0;
    s_ap[0] = 0;
  }
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int i = base + tid;
    int32_t ext = 0, np = 0;
    if (i < a.B) req_counts(a, req_fields(a, i), &ext, &np);
    int32_t v[kScanVals] = {ext, np, 0, 0, 0};
    int32_t ex[kScanVals], tot[kScanVals];
    block_scan(v, ex, tot, smem);
    if (i < a.B) {
      s_qo[i + 1] = carry_q + ex[0] + ext;
      s_ap[i + 1] = carry_a + ex[1] + np;
    }
    carry_q += tot[0];
    carry_a += tot[1];
  }
  __syncthreads();
  const int64_t t0 = (int64_t)(blockIdx.x - 1) * kMapTokens;
  if (tid < kMapTokens) {
    const int64_t t = t0 + tid;
    int32_t row = -1;
    if (t < a.T) row = map_token(a, t, s_qo, s_ap);
    s_rows[tid] = row;
  }
  if (!a.k_new) return;
  __syncthreads();
  const int rv = a.store_row_vec;
  const int n = kMapTokens * rv;
  for (int base = 0; base < n; base += kCopyVec * kPlanThreads) {
    uint4 kv[kCopyVec], vv[kCopyVec];
    int64_t dst[kCopyVec];
#pragma unroll
    for (int q = 0; q < kCopyVec; ++q) {
      const int idx = base + q * kPlanThreads + tid;
      const int k = idx / rv;
      const int c = idx - k * rv;
      // -1: past the block's vectors, past the batch's tokens, or a token that got no row
      const int32_t row = idx < n ? s_rows[min(k, kMapTokens - 1)] : -1;
      const int64_t src = row >= 0 ? (t0 + k) * rv + c : 0;
      kv[q] = row >= 0 ? a.k_new[src] : make_uint4(0, 0, 0, 0);
      vv[q] = row >= 0 ? a.v_new[src] : make_uint4(0, 0, 0, 0);
      dst[q] = row >= 0 ? (int64_t)row * a.store_stride_vec + c : -1;
    }
#pragma unroll
    for (int q = 0; q < kCopyVec; ++q) {
      if (dst[q] >= 0) {
        a.k_pool[dst[q]] = kv[q];
        a.v_pool[dst[q]] = vv[q];
      }
    }
  }
}

__global__ void __launch_bounds__(256) token_kernel(MetaArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.T) return;
  map_token(a, t, a.qo_indptr, (const int32_t*)(a.plan + a.layout.alloc_ptr_off));
}

__global__ void __launch_bounds__(kPlanThreads) plan_kernel(MetaArgs a) {
  __shared__ int32_t smem[kScanVals][kPlanWaves];
  if (blockIdx.x > 0) {  // a map block (uniform for the workgroup)
    __shared__ int32_t s_qo[kFuseReqs + 1];
    __shared__ int32_t s_ap[kFuseReqs + 1];
    __shared__ int32_t s_rows[kMapTokens];
    map_block(a, s_qo, s_ap, smem, s_rows);
    return;
  }
  const int tid = threadIdx.x;
  int32_t bits = 0;
  int32_t* header = (int32_t*)a.plan;
  int32_t* dec_tile_ptr = (int32_t*)(a.plan + a.layout.dec_tiles_off);
  int2* tiles = (int2*)(a.plan + a.layout.tiles_off);
  int2* tiles_raw = (int2*)(a.plan + a.layout.tiles_raw_off);
  int32_t* alloc_ptr = (int32_t*)(a.plan + a.layout.alloc_ptr_off);
  const int32_t s = a.page_shift;
  const int32_t tq = a.layout.tile_q;

  // Running totals and work lists, kPlanThreads requests at a time.
  int32_t carry[kScanVals] = {0, 0, 0, 0, 0};
  if (tid == 0) {
    a.qo_indptr[0] = 0;
    a.kv_indptr[0] = 0;
    dec_tile_ptr[0] = 0;
    alloc_ptr[0] = 0;
  }
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int i = base + tid;
    ReqInfo ri = {false, 0, 0, 0, 0, 0};  // valid, ext, dl, new_pages, dtiles, tiles
    if (i < a.B) {
      const ReqFields f = req_fields(a, i);
      if (i >= a.pad_from) {  // the later kernels read the padding from the arrays
        a.pad_table_idx[i] = f.r;
        a.pad_cached_len[i] = f.c;
        a.pad_device_len[i] = f.dl;
      }
      const int32_t dl = f.dl;
      ri.valid = request_ok(a, i, f, &bits);
      req_counts(a, f, &ri.ext, &ri.new_pages);
      ri.dl = dl > 0 ? dl : 0;
      if (ri.valid) {
        if (i < a.num_decode) ri.dtiles = (dl + kDecodeTileKeys - 1) / kDecodeTileKeys;
        else ri.tiles = (ri.ext + tq - 1) / tq;
      }
    }
    int32_t v[kScanVals] = {ri.ext, ri.dl, ri.new_pages, ri.dtiles, ri.tiles};
    int32_t ex[kScanVals], tot[kScanVals];
    block_scan(v, ex, tot, smem);
    if (i < a.B) {
      const int32_t qo_end = carry[0] + ex[0] + ri.ext;
      a.qo_indptr[i + 1] = qo_end;
      a.kv_indptr[i + 1] = carry[1] + ex[1] + ri.dl;
      a.last_indices[i] = qo_end - 1;
      alloc_ptr[i + 1] = carry[2] + ex[2] + ri.new_pages;
      // a padding request's one new page is the dummy page (its alloc entry,
      // for readers of alloc_rows; the token mapping knows it anyway)
      if (i >= a.pad_from && carry[2] + ex[2] < a.num_alloc) a.pad_alloc_rows[carry[2] + ex[2]] = 0;
      dec_tile_ptr[i + 1] = carry[3] + ex[3] + ri.dtiles;
      const int32_t tb = carry[4] + ex[4];
      const int32_t cap_t = a.layout.cap_tiles;
      for (int k = 0; k < ri.tiles && tb + k < cap_t; ++k) {
        // longest tiles (largest token offset, most keys) first
        tiles_raw[tb + k] = make_int2(i, (ri.tiles - 1 - k) * tq);
      }
    }
#pragma unroll
    for (int q = 0; q < kScanVals; ++q) carry[q] += tot[q];
  }
  if (tid == 0) {
    // the decode kernel's runs each take `per` consecutive tiles of the flat
    // (request, KV-head group, key tile) order
    const int32_t hg = decode_heads_per_group(a.Hkv);
    const int64_t runs = kDecodeWaves / hg;
    const int64_t total = (int64_t)(a.Hkv / hg) * carry[3];
    const int64_t per = total > 0 ? (total + runs - 1) / runs : 1;
    header[0] = (int32_t)total;
    header[1] = (int32_t)per;
    header[2] = min(carry[4], a.layout.cap_tiles);
    header[3] = tq;
    header[4] = (int32_t)((total + per - 1) / per);
    header[5] = a.layout.cap_tiles;
    if ((int64_t)carry[0] != a.T) bits |= PKV_STATUS_TOKEN_COUNT;
    if ((int64_t)carry[2] > a.num_alloc) bits |= PKV_STATUS_BAD_ALLOC;
  }
  if (bits) raise_status(a.status, bits);

  // Extend tiles by key count, most first: a counting sort over kSortBuckets
  // buckets of 64 keys.  Workgroups start in list order, so the longest run
  // first and the shortest fill the last gaps (longest-processing-time
  // order).  The order inside a bucket is whatever the LDS atomics give;
  // every tile's result is independent of it.
  __shared__ int32_t bucket[kSortBuckets];
  const int32_t n_t = min(carry[4], a.layout.cap_tiles);  // the same in every thread
  if (n_t > 0) {  // decode-only batches skip the sort
    auto tile_bucket = [&](int2 t) -> int {
      const ReqFields f = req_fields(a, t.x);
      const int32_t ci = f.c;
      const int32_t di = f.dl;
      const int32_t kv_end = min(di, ci + t.y + tq);
      return kSortBuckets - 1 - min(max(kv_end, 0) >> 6, kSortBuckets - 1);
    };
    for (int b = tid; b < kSortBuckets; b += kPlanThreads) bucket[b] = 0;
    __syncthreads();  // also orders the tiles_raw writes above before the reads below
    for (int t = tid; t < n_t; t += kPlanThreads) atomicAdd(&bucket[tile_bucket(tiles_raw[t])], 1);
    __syncthreads();
    {
      constexpr int kPer = kSortBuckets / kPlanThreads;
      int32_t cnt[kPer];
      int32_t mine = 0;
  #pragma unroll
      for (int q = 0; q < kPer; ++q) {
        cnt[q] = bucket[tid * kPer + q];
        mine += cnt[q];
      }
      int32_t v[kScanVals] = {mine, 0, 0, 0, 0};
      int32_t ex[kScanVals], tot[kScanVals];
      block_scan(v, ex, tot, smem);
      int32_t run = ex[0];
  #pragma unroll
      for (int q = 0; q < kPer; ++q) {
        bucket[tid * kPer + q] = run;  // first position of the bucket
        run += cnt[q];
      }
    }
    __syncthreads();
    for (int t = tid; t < n_t; t += kPlanThreads) {
      const int2 tt = tiles_raw[t];
      tiles[atomicAdd(&bucket[tile_bucket(tt)], 1)] = tt;
    }
  }
}

MetaArgs metadata_launch_args(const MetaArgs& a_in) {
  MetaArgs a = a_in;
  a.map_blocks = (a.B <= kFuseReqs && a.T > 0) ? (int32_t)((a.T + kMapTokens - 1) / kMapTokens) : 0;
  return a;
}

}  // namespace

hipError_t launch_metadata(const MetaArgs& a_in, hipStream_t s) {
  const MetaArgs a = metadata_launch_args(a_in);
  hipLaunchKernelGGL(plan_kernel, dim3(1 + a.map_blocks), dim3(kPlanThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.T == 0 || a.map_blocks > 0) return e;
  const int64_t blocks = (a.T + 255) / 256;
  hipLaunchKernelGGL(token_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

bool metadata_stores_rows(const MetaArgs& a) { return a.k_new && metadata_launch_args(a).map_blocks > 0; }

void metadata_plan_node(const MetaArgs& a, MetaArgs* args, void** argv, hipKernelNodeParams* p) {
  *args = metadata_launch_args(a);
  argv[0] = args;
  p->func = reinterpret_cast<void*>(plan_kernel);
  p->gridDim = dim3(1 + args->map_blocks);
  p->blockDim = dim3(kPlanThreads);
  p->sharedMemBytes = 0;
  p->kernelParams = argv;
  p->extra = nullptr;
}

}  // namespace pkv
