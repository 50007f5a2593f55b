/*
 * pagedkv.h - C ABI of the MI355X (gfx950) paged-KV attention step of one
 * transformer layer.
 *
 * The step follows the Req/Batch model described in "mini-sglang learning
 * notes" (doc-mini-sglang-learn: the Req, Batch, KV-pool, page-table,
 * store_kv and dummy-page passages) and "mini-sglang architecture deep dive"
 * (tinymind.me) sections 5.1-5.3 and 6.2:
 *
 *   build_attn_metadata  page-table write for the batch's new tokens, out_loc,
 *                        positions, running totals, and the attention plan
 *   kv_store             scatter of the new K/V rows to their out_loc rows
 *   paged_decode_attn    split-K decode attention (one new token per request)
 *   paged_extend_attn    chunked-prefill attention on a cached prefix
 * and around them:
 *   build_attn_metadata_store  the first two in one launch (up to 1024 requests)
 *   paged_decode_attn_static   decode attention that allocates nothing
 *   kv_store_rope        kv_store with rotary position embedding (and an
 *                        optional per-head RMS norm) applied to q and k on
 *                        the way (deep dive sections 7.2-7.3)
 *   pkv_alloc_pages / pkv_free_pages   the page free list on the device
 *   pkv_decode_graph_*   the decode step captured as HIP graphs
 *   pkv_kv_cache_layer   one layer of a multi-layer KV cache
 *   pkv_plan_view_layout where the plan keeps its work lists
 *
 * Conventions shared by every entry point
 *   - Every pointer inside the structs and every data argument is a DEVICE
 *     pointer unless marked "host".  The structs themselves are read on the
 *     host during the call and may be freed when it returns.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises; it only enqueues kernels on `stream` (a hipStream_t,
 *     passed as void*; NULL means the legacy default stream).  All calls are
 *     asynchronous, stateless and reentrant, so they can be captured in a
 *     HIP graph when the buffers keep fixed addresses.
 *   - Return codes are checked on the host BEFORE any launch: on a non-zero
 *     return nothing was enqueued (except PKV_ERR_HIP, which reports a
 *     launch failure).  Values that live on the device (lengths, table
 *     indices, out_loc, page-table entries) cannot be checked on the host;
 *     kernels check each one before using it as an address, skip the
 *     offending request / token / key, and OR a PKV_STATUS_* bit into the
 *     caller's `status` word (if non-NULL).  A bad device value therefore
 *     never causes an out-of-bounds access.
 *   - bf16 is IEEE bfloat16; outputs are rounded from fp32 to nearest even.
 *   - head_dim must be 128; query heads per KV head (Hq / Hkv) must be 1..16.
 *     Consecutive query heads share a KV head: query head h reads KV head
 *     h / (Hq / Hkv).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes (host side) ------------------------------------------ */
#define PKV_OK                    0
#define PKV_ERR_INVALID_ARGUMENT  1  /* null pointer, negative size, bad stride or shape relation */
#define PKV_ERR_UNSUPPORTED       2  /* head_dim != 128, Hq/Hkv outside 1..16, page_size not a power of two <= 64 */
#define PKV_ERR_WORKSPACE         3  /* plan or workspace smaller than the size query returns */
#define PKV_ERR_HIP               4  /* a kernel launch failed; see pkv_last_hip_error() */
#define PKV_ERR_HOST_ALLOC        5  /* a host allocation failed (pkv_decode_graph_create only) */
#define PKV_ERR_SCRATCH           6  /* the call needs more than the library's static scratch holds */

/* ---- device status bits (sticky; OR-ed into *status by kernels) ---------- */
#define PKV_STATUS_BAD_OUT_LOC    0x01  /* out_loc[t] outside [0, num_rows): token skipped by kv_store */
#define PKV_STATUS_BAD_LENGTHS    0x02  /* not 0 <= cached_len <= device_len <= W: request skipped */
#define PKV_STATUS_BAD_TABLE_IDX  0x04  /* table_idx outside [0, R): request skipped */
#define PKV_STATUS_BAD_PAGE_ROW   0x08  /* a page-table entry or new row outside the pool: key or token skipped */
#define PKV_STATUS_BAD_DECODE     0x10  /* a request below num_decode whose extend_len != 1: skipped */
#define PKV_STATUS_TOKEN_COUNT    0x20  /* sum of extend_len differs from num_tokens */
#define PKV_STATUS_BAD_ALLOC      0x40  /* alloc_rows entry misaligned, outside the pool, or too few entries */
#define PKV_STATUS_BAD_POSITION   0x80  /* positions[t] outside [0, max_position): token skipped by kv_store_rope */
#define PKV_STATUS_OUT_OF_PAGES   0x100 /* the free list held fewer pages than the batch needs: nothing allocated */
#define PKV_STATUS_FREE_OVERFLOW  0x200 /* freeing would overfill the free list: nothing freed */

/* ---- data structures ---------------------------------------------------- */

/* One layer's KV pool (learning notes, KV-pool passage; deep dive 6.2): each
 * of K and V is an array of token rows of shape (pages * page_size, kv_heads,
 * head_dim), and a token's physical position is simply its row number.
 * Element (row r, KV head g, dim e) of K is at k + (r*row_stride + g*head_dim + e)
 * bf16 elements; the same for V.  Page p owns rows [p*page_size, (p+1)*page_size). */
typedef struct pkv_kv_pool {
  void*   k;             /* bf16 K rows */
  void*   v;             /* bf16 V rows */
  int64_t num_rows;      /* rows in the pool; a multiple of page_size, < 2^31 */
  int64_t row_stride;    /* bf16 elements from one row to the next; >= num_kv_heads*head_dim, multiple of 8, < 2^31 */
  int32_t page_size;     /* 1, 2, 4, ..., 64 */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* d; must be 128 */
  int32_t reserved;      /* must be 0 */
} pkv_kv_pool;

/* page_table (learning notes, page-table passage): one row per request slot
 * (table_idx); column j holds the RAW physical pool row of logical token j;
 * the width is aligned up to 32.  int32 [num_rows, width], row-major. */
typedef struct pkv_page_table {
  int32_t* data;
  int32_t  num_rows;     /* R */
  int32_t  width;        /* W; a positive multiple of 32 */
} pkv_page_table;

/* The batch (learning notes, Req and Batch passages).  For request i:
 * cached_len = tokens already in the pool, device_len = tokens covered after
 * this forward, extend_len = device_len - cached_len new tokens.  The new
 * tokens of all requests are laid out in request order ("batch order"): q, o,
 * k_new, v_new, out_loc and positions all have one row per new token in that
 * order.  The first num_decode requests are decode requests (extend_len == 1);
 * the rest are extend requests.  Padding requests (CUDA-graph-style batch
 * filling) are ordinary decode requests with cached_len 0, device_len 1 and a
 * table row whose entries all point at the dummy page. */
typedef struct pkv_batch {
  int32_t        num_reqs;    /* B >= 0 */
  int32_t        num_decode;  /* 0 <= num_decode <= B */
  int64_t        num_tokens;  /* T = sum of extend_len (host-known; sizes the per-token arrays) */
  const int32_t* table_idx;   /* [B] page-table row of each request */
  const int32_t* cached_len;  /* [B] */
  const int32_t* device_len;  /* [B] */
} pkv_batch;

/* Per-batch metadata, written by build_attn_metadata into caller-owned
 * buffers (fixed addresses allow graph replay) and read by the attention
 * calls of every layer of that batch. */
typedef struct pkv_attn_metadata {
  int32_t* out_loc;       /* [T]   physical pool row of each new token */
  int32_t* positions;     /* [T]   logical position (cached_len + offset) of each new token */
  int32_t* qo_indptr;     /* [B+1] running total of extend_len, starting at 0 */
  int32_t* kv_indptr;     /* [B+1] running total of device_len, starting at 0 */
  int32_t* last_indices;  /* [B]   qo_indptr[i+1] - 1: row of each request's last new token */
  void*    plan;          /* opaque work lists for the attention kernels */
  size_t   plan_bytes;    /* >= pkv_plan_bytes(B, T, Hq, Hkv) */
  int32_t* status;        /* [1] sticky PKV_STATUS_* bits, or NULL */
} pkv_attn_metadata;

/* ---- size queries (pure host functions) --------------------------------- */

/* Bytes of pkv_attn_metadata.plan for batches of at most max_reqs requests and
 * max_tokens new tokens with these head counts.  0 on invalid arguments. */
size_t pkv_plan_bytes(int32_t max_reqs, int64_t max_tokens, int32_t num_qo_heads, int32_t num_kv_heads);

/* Bytes of the workspace paged_decode_attn needs (the split-K partial
 * results: fp32 accumulators plus running max and sum of the pieces of
 * requests that several runs of wavefronts share).  It does not depend on max_reqs
 * (kept for the ABI): about 34 MB at most.  0 on invalid arguments. */
size_t paged_attn_workspace_bytes(int32_t max_reqs, int32_t num_qo_heads, int32_t head_dim);

/* ---- entry points ------------------------------------------------------- */

/* kv_store: K[out_loc[t]] = k_new[t] and V[out_loc[t]] = v_new[t] for
 * t < num_tokens (learning notes, store_kv passage: each layer first scatters
 * the batch's new K/V to the out_loc physical positions; the dummy page
 * absorbs padding writes).
 *   k_new, v_new : bf16 [num_tokens, Hkv, head_dim], contiguous
 *   out_loc      : int32 [num_tokens]
 * Tokens with the same target row (only padding tokens on the dummy page)
 * race: that row ends up holding one of them, possibly mixed.  A token whose
 * out_loc is outside the pool is skipped (PKV_STATUS_BAD_OUT_LOC), except -1,
 * build_attn_metadata's mark for a token it could not map, which is skipped
 * silently (the cause is already reported).
 * num_tokens == 0 is a no-op. */
int kv_store(const pkv_kv_pool* pool, const void* k_new, const void* v_new, const int32_t* out_loc,
             int64_t num_tokens, int32_t* status, void* stream);

/* build_attn_metadata: for each request i and each new logical position
 * j in [cached_len, device_len) (learning notes, page-table passage: page
 * aligned allocation over [cached_len, device_len) from free_slots, written
 * back with the raw physical rows):
 *   - if j lies in the request's partially filled last cached page,
 *       row = page_table[r, j - j % s] + j % s
 *     otherwise it lies in the request's k-th new page and
 *       row = alloc_rows[first new page of i + k] + j % s;
 *   - page_table[table_idx[i], j] = row;  out_loc[t] = row;  positions[t] = j;
 * and writes qo_indptr, kv_indptr, last_indices and the attention plan.
 *   page_size  : s of the pool (a power of two <= 64)
 *   num_pool_rows : rows of the pool (alloc rows + j % s must stay below it)
 *   alloc_rows : int32 [num_alloc], the first pool row (a multiple of s) of
 *                every newly allocated page, request by request; request i
 *                takes ceil(device_len/s) - ceil(cached_len/s) pages.  With
 *                s == 1 this is exactly out_loc.
 *   num_qo_heads, num_kv_heads : head counts the plan is built for; the
 *                attention calls must use the same ones.
 * Requests with invalid lengths or table_idx are skipped (status bit set);
 * entries outside [cached_len, device_len) of each row are left untouched.
 * A token that gets no row (its request skipped, a bad alloc or page-table
 * entry, or past the batch's real tokens) has out_loc and positions set to
 * -1, which kv_store and kv_store_rope skip. */
int build_attn_metadata(const pkv_batch* batch, const pkv_page_table* page_table, int32_t page_size,
                        int64_t num_pool_rows, const int32_t* alloc_rows, int64_t num_alloc,
                        int32_t num_qo_heads, int32_t num_kv_heads, const pkv_attn_metadata* meta,
                        void* stream);

/* build_attn_metadata_store: build_attn_metadata followed by kv_store of the
 * batch's new K/V rows at the out_loc rows it writes (the order the learning
 * notes' store_kv passage gives: rows are placed before attention reads
 * them), with identical results, in fewer launches: for a batch of at most
 * 1024 requests (every configuration here) one launch does both, its extra
 * workgroups mapping 8 tokens each and copying their rows while the first
 * builds the metadata; larger batches take the two calls' launches.  The
 * pool's page_size and num_rows stand for
 * build_attn_metadata's page_size and num_pool_rows, its num_kv_heads for
 * num_kv_heads.
 *   k_new, v_new : bf16 [num_tokens, Hkv, head_dim], contiguous, 16-byte aligned
 * Tokens that get no row (out_loc -1) are not stored; padding tokens sharing
 * the dummy row race as in kv_store.  Errors as the two calls'. */
int build_attn_metadata_store(const pkv_batch* batch, const pkv_page_table* page_table, const pkv_kv_pool* pool,
                              const int32_t* alloc_rows, int64_t num_alloc, int32_t num_qo_heads,
                              const pkv_attn_metadata* meta, const void* k_new, const void* v_new, void* stream);

/* paged_decode_attn: for each decode request i < num_decode and query head h,
 *   o[qo_indptr[i], h] = softmax(sm_scale * q[qo_indptr[i], h] . K[rows]^T) V[rows]
 * over rows = page_table[table_idx[i], 0 .. device_len[i]) (the new row stored
 * by kv_store included), gathered through the page table.  Split-K over the
 * keys (learning notes kernel passage; flash-decoding):
 * the (request, group of KV heads, 32-key tile) work is split evenly over a
 * fixed set of runs of wavefronts, so a request's keys may be shared by
 * several of them, and a merge kernel combines their partial softmax states.
 *   q, o       : bf16 [num_tokens, Hq, head_dim]; rows of extend requests untouched
 *   workspace  : >= paged_attn_workspace_bytes(B, Hq, head_dim) bytes, 16-byte aligned
 * Must follow build_attn_metadata (same batch, head counts) and kv_store on
 * the same stream (or be ordered after them). */
int paged_decode_attn(const pkv_kv_pool* pool, const pkv_page_table* page_table, const pkv_batch* batch,
                      const pkv_attn_metadata* meta, const void* q, void* o, int32_t num_qo_heads,
                      float sm_scale, void* workspace, size_t workspace_bytes, void* stream);

/* paged_extend_attn: chunked prefill on a cached prefix (learning notes,
 * Req and chunked-prefill passages; deep dive 5.2).  For each extend request
 * i >= num_decode and its new token t (position p = cached_len + t) and query
 * head h,
 *   o[qo_indptr[i] + t, h] = softmax(sm_scale * q . K[rows 0..p]^T) V[rows 0..p]
 * i.e. the whole cached prefix is visible and the new rows are causal.
 * QK^T and PV run on bf16 MFMA with fp32 accumulation; the probabilities are
 * rounded to bf16 before PV.
 *   q, o : bf16 [num_tokens, Hq, head_dim]; rows of decode requests untouched
 *   workspace : unused (may be NULL)
 * Same ordering requirements as paged_decode_attn. */
int paged_extend_attn(const pkv_kv_pool* pool, const pkv_page_table* page_table, const pkv_batch* batch,
                      const pkv_attn_metadata* meta, const void* q, void* o, int32_t num_qo_heads,
                      float sm_scale, void* workspace, size_t workspace_bytes, void* stream);

/* paged_decode_attn_static: paged_decode_attn without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The split-K
 * partial states go to a static device array of PKV_STATIC_SCRATCH_BYTES bytes
 * inside the library; the call allocates nothing (no hipMalloc / hipFree).
 * Each GPU the library runs on holds its own copy of the array until the
 * process ends; the first call on a device looks up its address there.
 * Limit: the array holds the partial states of up to 8 query heads per KV head
 * (Hq / Hkv <= 8); a larger group returns PKV_ERR_SCRATCH before anything is
 * enqueued.  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other threads) race, so the caller serialises
 * them (one stream, or events between streams).  The array needs no clearing
 * between calls: every partial state the merge reads is written earlier in the
 * same call.  Results are bit-identical to paged_decode_attn's on the same
 * inputs. */
#define PKV_STATIC_SCRATCH_BYTES 17039360  /* 2048 wavefronts x 2 pieces x 8 heads x (128 + 2) floats */
int paged_decode_attn_static(const pkv_kv_pool* pool, const pkv_page_table* page_table, const pkv_batch* batch,
                             const pkv_attn_metadata* meta, const void* q, void* o, int32_t num_qo_heads,
                             float sm_scale, void* stream);

/* ---- all layers' KV cache in one buffer ------------------------------------ */

/* The engine's KV cache (deep dive 6.2, MHAKVCache): one bf16 buffer holding K
 * (index 0) and V (index 1) of every layer.  Three physical orders:
 *   PKV_LAYOUT_LAYER_FIRST : [2][num_layers][num_rows][Hkv][head_dim]
 *                            (a layer's rows are contiguous)
 *   PKV_LAYOUT_PAGE_FIRST  : [2][num_rows][num_layers][Hkv][head_dim]
 *                            (a row's layers are contiguous; the pages' permuted
 *                            view has the same logical shape, but a layer's rows
 *                            are num_layers * Hkv * head_dim elements apart)
 *   PKV_LAYOUT_ROW_INTERLEAVED : [num_rows][num_layers][2][Hkv][head_dim]
 *                            (a row's K and V of every layer are contiguous,
 *                            so a gathered row's K and V lie on one memory
 *                            page: half the address translations of separate
 *                            K and V buffers when rows are scattered)
 * Every call works on one layer's pkv_kv_pool, obtained with pkv_kv_cache_layer. */
#define PKV_LAYOUT_LAYER_FIRST     0
#define PKV_LAYOUT_PAGE_FIRST      1
#define PKV_LAYOUT_ROW_INTERLEAVED 2

typedef struct pkv_kv_cache {
  void* data;              /* device, 16-byte aligned */
  int64_t num_rows;        /* pages * page_size, < 2^31 */
  int32_t num_layers;      /* > 0 */
  int32_t layout;          /* PKV_LAYOUT_* */
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t reserved;        /* must be 0 */
} pkv_kv_cache;

/* pkv_kv_cache_layer: fills *pool (host struct) with layer layer_id's K and V
 * base pointers and row stride (the forward pass's layer_id, deep dive 5.1).
 * Host only; launches nothing. */
int pkv_kv_cache_layer(const pkv_kv_cache* cache, int32_t layer_id, pkv_kv_pool* pool);

/* ---- rotary position embedding fused into the store ----------------------- */

/* Optional RMS norm of every q and k head row before the rotation (deep dive
 * 7.2: models such as Qwen3 normalise q and k per head):
 *   x <- x / sqrt(mean(x^2) + eps) * weight, over the head_dim elements.
 * The normalised row is rotated without an intermediate bf16 rounding. */
typedef struct pkv_qk_norm {
  const void* q_weight;  /* bf16 [head_dim] */
  const void* k_weight;  /* bf16 [head_dim] */
  float eps;             /* >= 0 */
  int32_t reserved;      /* must be 0 */
} pkv_qk_norm;

/* pkv_rope_cos_sin_cache: the rotary table of deep dive 7.3 (rotary_dim equal
 * to head_dim, inverse frequencies theta_i = base^(-2i/head_dim)):
 *   cache[p * head_dim + i]              = cos(p * theta_i)
 *   cache[p * head_dim + head_dim/2 + i] = sin(p * theta_i)
 * for p < max_position and i < head_dim/2.  Angles are formed in float64 and
 * the values rounded to float.
 *   cache : float [max_position, head_dim], caller-owned, 16-byte aligned
 * Built once per model; head_dim must be 128, base > 1. */
int pkv_rope_cos_sin_cache(float* cache, int32_t max_position, int32_t head_dim, double base, void* stream);

/* kv_store_rope: for each token t < num_tokens with p = positions[t]
 * (deep dive 7.2-7.3: the attention layer rotates q and k by position, then
 * the backend stores K/V):
 *   every q head row and k head row x (optionally RMS-normed first) becomes
 *     y_j          = x_j * cos(p theta_j) - x_{j+d/2} * sin(p theta_j)
 *     y_{j+d/2}    = x_{j+d/2} * cos(p theta_j) + x_j * sin(p theta_j)
 *   (the "rotate half" pairing, j < d/2, cos/sin read from the table);
 *   q is rotated in place, the rotated k goes to K[out_loc[t]] and v_new[t]
 *   to V[out_loc[t]] unchanged.
 *   q            : bf16 [num_tokens, num_qo_heads, head_dim], in/out
 *   k_new, v_new : bf16 [num_tokens, Hkv, head_dim]
 *   out_loc, positions : int32 [num_tokens] (positions as build_attn_metadata writes them)
 *   cos_sin_cache : float [max_position, head_dim] from pkv_rope_cos_sin_cache
 *   qk_norm      : NULL for no norm (host struct, device weights)
 * All rows 16-byte aligned and contiguous.  A token whose position is outside
 * [0, max_position) is left entirely untouched (PKV_STATUS_BAD_POSITION); one
 * whose out_loc is outside the pool has q rotated but nothing stored
 * (PKV_STATUS_BAD_OUT_LOC).  A position or out_loc of -1 (an unmapped token)
 * is skipped the same way without raising a bit.  Tokens sharing a target row race as in kv_store.
 * num_tokens == 0 is a no-op. */
int kv_store_rope(const pkv_kv_pool* pool, void* q, int32_t num_qo_heads, const void* k_new, const void* v_new,
                  const int32_t* out_loc, const int32_t* positions, int64_t num_tokens,
                  const float* cos_sin_cache, int32_t max_position, const pkv_qk_norm* qk_norm,
                  int32_t* status, void* stream);

/* ---- page allocator on the GPU ------------------------------------------- */

/* A free list of page-start rows kept on the device as a ring (learning
 * notes, page-table passage: free_slots, page aligned; deep dive 3.6: freed
 * entries are appended).  The oldest free page is rows[state[0]]; state[1]
 * pages are free, at ring positions state[0], state[0] + 1, ... (mod
 * capacity).  Concurrent calls on one free list race. */
typedef struct pkv_free_list {
  int32_t* rows;           /* int32 [capacity], device */
  int32_t* state;          /* int32 [2], device: head, number of free pages */
  int32_t capacity;        /* > 0 */
  int32_t page_size;       /* a power of two <= 64; every row is a multiple of it */
  int64_t num_pool_rows;   /* rows of the pool the pages belong to */
} pkv_free_list;

/* pkv_free_list_reset: the caller has written num_free page-start rows to
 * rows[0, num_free); sets head 0 and num_free free pages (0 <= num_free <= capacity). */
int pkv_free_list_reset(const pkv_free_list* free_list, int32_t num_free, void* stream);

/* pkv_alloc_pages: request i of the batch needs
 *   ceil(device_len/s) - ceil(cached_len/s) pages (0 unless 0 <= cached_len <= device_len),
 * the page-aligned count over [cached_len, device_len); the batch takes the
 * next n = sum of them oldest-first, request by request, into alloc_rows[0, n)
 * (the alloc_rows input of build_attn_metadata for the same batch), and the
 * list loses them.  If fewer than n are free, or n > max_alloc, nothing is
 * taken, alloc_rows[0, min(n, max_alloc)) are set to -1 (build_attn_metadata
 * then maps none of the batch's new tokens) and PKV_STATUS_OUT_OF_PAGES is
 * raised: the caller evicts and retries.  A row that is not page aligned or
 * outside the pool is passed on and raises PKV_STATUS_BAD_ALLOC. */
int pkv_alloc_pages(const pkv_free_list* free_list, const pkv_batch* batch, int32_t* alloc_rows, int64_t max_alloc,
                    int32_t* status, void* stream);

/* pkv_free_pages: appends rows[0, num_rows) (device, page-start rows) to the
 * free list in order.  Nothing is freed if one of them is not a page-aligned
 * row of the pool (PKV_STATUS_BAD_ALLOC) or the list would exceed its
 * capacity (PKV_STATUS_FREE_OVERFLOW). */
int pkv_free_pages(const pkv_free_list* free_list, const int32_t* rows, int32_t num_rows, int32_t* status,
                   void* stream);

/* ---- decode step as HIP graphs ------------------------------------------ */

/* The fixed buffers of a graph-replayed decode step (deep dive 4.3, learning
 * notes graph passage: every input, output and workspace keeps the address it
 * had at capture).  All device pointers, sized for max_reqs requests (one
 * token each): */
typedef struct pkv_decode_graph_desc {
  pkv_kv_pool pool;
  pkv_page_table page_table;
  int32_t max_reqs;
  int32_t dummy_table_row;     /* an all-zero page-table row: padding requests use it */
  int32_t num_qo_heads;
  float sm_scale;
  int32_t* table_idx;          /* int32 [max_reqs] */
  int32_t* cached_len;         /* int32 [max_reqs] */
  int32_t* device_len;         /* int32 [max_reqs] */
  int32_t* alloc_rows;         /* int32 [max_reqs]: new-page rows, as for build_attn_metadata */
  const void* q;               /* bf16 [max_reqs, Hq, head_dim] */
  void* o;                     /* bf16 [max_reqs, Hq, head_dim] */
  const void* k_new;           /* bf16 [max_reqs, Hkv, head_dim] */
  const void* v_new;           /* bf16 [max_reqs, Hkv, head_dim] */
  pkv_attn_metadata meta;      /* buffers for (max_reqs requests, max_reqs tokens) */
  void* workspace;             /* >= paged_attn_workspace_bytes(max_reqs, Hq, head_dim) */
  size_t workspace_bytes;
  int32_t reserved;            /* must be 0 */
} pkv_decode_graph_desc;

typedef struct pkv_decode_graph pkv_decode_graph;  /* opaque, host side */

/* pkv_decode_graph_create: capture, for each batch size in sizes (host array,
 * strictly increasing, each <= max_reqs; the pages' list is 1, 2, 4, 8, 16, ...),
 * one graph of build_attn_metadata_store (metadata, then the rows at its
 * out_loc) -> paged_decode_attn on a decode batch of that many requests in desc's
 * buffers.  stream must be a non-default stream (capture happens on it; the
 * buffers' contents are not read during capture).  This is the one call that
 * allocates: host memory and the graphs' driver objects, no device memory,
 * released by pkv_decode_graph_destroy.  A failing host check of any of the
 * three calls is returned and nothing is kept; PKV_ERR_HOST_ALLOC if the
 * graph object cannot be allocated. */
int pkv_decode_graph_create(const pkv_decode_graph_desc* desc, const int32_t* sizes, int32_t num_sizes,
                            pkv_decode_graph** graph, void* stream);

/* pkv_decode_graph_replay: the caller has written its num_reqs real decode
 * requests into slots [0, num_reqs) of table_idx / cached_len / device_len /
 * q / k_new / v_new and their new-page rows into alloc_rows, request by
 * request from entry 0 (one entry per page a request needs; with page_size 1
 * exactly num_reqs entries).  The call picks the smallest captured size
 * bs >= num_reqs (written to *graph_size if non-NULL) and launches that graph
 * on stream, with num_reqs set in its first kernel: that kernel turns slots
 * [num_reqs, bs) into dummy requests on dummy_table_row (cached_len 0,
 * device_len 1, their one new row the dummy page's row 0, written to those
 * slots of table_idx / cached_len / device_len) and counts the real
 * requests' new pages on the device, so alloc_rows[num_reqs..] is not read.
 * One launch per replay.  Outputs of the real requests are in o[0, num_reqs).
 * Replays on one graph object must not overlap. */
int pkv_decode_graph_replay(pkv_decode_graph* graph, int32_t num_reqs, int32_t* graph_size, void* stream);

int pkv_decode_graph_destroy(pkv_decode_graph* graph);

/* ---- plan inspection (diagnostics and tests) ------------------------------ */

/* Where the plan that build_attn_metadata writes (for batches of at most
 * max_reqs requests and max_tokens new tokens, these head counts) keeps the
 * work lists the attention calls follow.  The plan stays opaque to the calls;
 * this lets a caller copy it to the host and check that the work lists cover
 * every (request, KV head, key) of the decode requests and every (request, new
 * token) of the extend requests exactly once.  Offsets are bytes from the
 * start of the plan.
 *   header, int32[8]:
 *     [0] decode tiles in the flat order (see below)
 *     [1] decode tiles per run ("per")
 *     [2] extend tiles listed
 *     [3] new tokens per extend tile (extend_tile_tokens)
 *     [4] decode runs that received tiles
 *   decode_tile_ptr, int32[B+1]: running total of the decode tiles of each
 *     request in one group's sequence: ceil(device_len / decode_tile_keys) for
 *     a valid decode request, 0 for extend and invalid requests.
 *   extend_tiles, int32 pairs [header[2]]: (request, first new-token offset);
 *     a tile covers new tokens [offset, offset + extend_tile_tokens) of the
 *     request (clipped to its extend_len), for every KV head.
 * The decode split (flash-decoding over the keys, learning notes kernel
 * passage): the flat order is request-major, then group of
 * decode_group_heads consecutive KV heads, then 32-key tile; with
 * Hg = Hkv / decode_group_heads groups, request i's group gg holds flat tiles
 * Hg * decode_tile_ptr[i] + gg * n_i + [0, n_i), n_i its tile count, and flat
 * tile kti of it covers keys [32 kti, min(32 kti + 32, device_len)) of the
 * group's KV heads.  Run r (of decode_runs) takes flat tiles
 * [r * per, min((r + 1) * per, header[0])).
 * Returns PKV_ERR_INVALID_ARGUMENT / PKV_ERR_UNSUPPORTED as pkv_plan_bytes
 * would return 0.  Host only. */
typedef struct pkv_plan_view {
  int64_t header_offset;
  int64_t decode_tile_ptr_offset;
  int64_t extend_tiles_offset;
  int64_t total_bytes;           /* == pkv_plan_bytes(...) */
  int32_t decode_runs;           /* runs the decode split spreads the flat order over */
  int32_t decode_group_heads;    /* KV heads one run reads together */
  int32_t decode_tile_keys;      /* keys per decode tile (32) */
  int32_t extend_tile_tokens;    /* new tokens per extend tile */
} pkv_plan_view;

int pkv_plan_view_layout(int32_t max_reqs, int64_t max_tokens, int32_t num_qo_heads, int32_t num_kv_heads,
                         pkv_plan_view* view);

/* ---- diagnostics -------------------------------------------------------- */
const char* pkv_error_string(int code);   /* static string, never NULL */
int         pkv_last_hip_error(void);      /* hipError_t of the last PKV_ERR_HIP in this thread */
int         pkv_version(void);             /* ABI version: 2 */

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
