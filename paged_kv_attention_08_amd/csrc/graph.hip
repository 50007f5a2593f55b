// pkv_decode_graph_*: the decode step (build_attn_metadata -> kv_store ->
// paged_decode_attn) captured once per padded batch size into HIP graphs and
// replayed with one launch.
//
// mini-sglang architecture deep dive, section 4.3 (GraphRunner: one graph per
// batch size in a list, captured on a batch of dummy requests; a decode batch
// no larger than the largest size is padded to its size and that graph is
// replayed) and the learning notes' graph passage (default sizes 1, 2, 4 and
// then multiples of 8; replay needs every input, output and workspace at the
// address it had during capture, and the attention plan re-made into fixed
// buffers).  Here the plan is built on the GPU by build_attn_metadata inside
// the graph, so a replay re-plans with no host work: the host only writes the
// real requests into the fixed buffers, one small kernel turns the remaining
// slots into dummy requests, and the graph is launched.
#include <algorithm>
#include <new>
#include <vector>

#include "kernels.hpp"

struct pkv_decode_graph {
  pkv_decode_graph_desc desc;
  std::vector<int32_t> sizes;          // ascending
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
};

namespace pkv {
namespace {

// Slots [n_real, bs) become dummy requests: the all-zero page-table row, no
// cached token, one new token whose row is the dummy page's first row.  Their
// alloc entries (one page each) follow the real requests' entries.
__global__ void __launch_bounds__(256) pad_kernel(int32_t* table_idx, int32_t* cached_len, int32_t* device_len,
                                                  int32_t* alloc_rows, int32_t n_real, int32_t bs,
                                                  int32_t n_alloc_real, int32_t dummy_row) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (n_real + k >= bs) return;
  table_idx[n_real + k] = dummy_row;
  cached_len[n_real + k] = 0;
  device_len[n_real + k] = 1;
  alloc_rows[n_alloc_real + k] = 0;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

namespace {

// The step on a batch of bs decode requests, enqueued on s (captured by the caller).
int enqueue_step(const pkv_decode_graph_desc& d, int32_t bs, hipStream_t s) {
  pkv_batch b;
  b.num_reqs = bs;
  b.num_decode = bs;
  b.num_tokens = bs;
  b.table_idx = d.table_idx;
  b.cached_len = d.cached_len;
  b.device_len = d.device_len;
  int rc = build_attn_metadata(&b, &d.page_table, d.pool.page_size, d.pool.num_rows, d.alloc_rows, bs,
                               d.num_qo_heads, d.pool.num_kv_heads, &d.meta, s);
  if (rc != PKV_OK) return rc;
  rc = kv_store(&d.pool, d.k_new, d.v_new, d.meta.out_loc, bs, d.meta.status, s);
  if (rc != PKV_OK) return rc;
  return paged_decode_attn(&d.pool, &d.page_table, &b, &d.meta, d.q, d.o, d.num_qo_heads, d.sm_scale, d.workspace,
                           d.workspace_bytes, s);
}

void release(pkv_decode_graph* g) {
  for (hipGraphExec_t e : g->execs)
    if (e) (void)hipGraphExecDestroy(e);
  for (hipGraph_t gr : g->graphs)
    if (gr) (void)hipGraphDestroy(gr);
  delete g;
}

}  // namespace

extern "C" {

int pkv_decode_graph_create(const pkv_decode_graph_desc* desc, const int32_t* sizes, int32_t num_sizes,
                            pkv_decode_graph** out, void* stream) {
  if (!desc || !sizes || num_sizes <= 0 || !out || !stream) return PKV_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  const pkv_decode_graph_desc& d = *desc;
  if (d.max_reqs <= 0 || !d.table_idx || !d.cached_len || !d.device_len || !d.alloc_rows || !d.k_new || !d.v_new ||
      !d.q || !d.o || d.reserved != 0)
    return PKV_ERR_INVALID_ARGUMENT;
  if (d.dummy_table_row < 0 || d.dummy_table_row >= d.page_table.num_rows) return PKV_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < num_sizes; ++i)
    if (sizes[i] <= 0 || sizes[i] > d.max_reqs || (i > 0 && sizes[i] <= sizes[i - 1])) return PKV_ERR_INVALID_ARGUMENT;
  // the calls check everything else on the host during capture (a failed
  // check ends the capture and is returned)
  pkv_decode_graph* g = new (std::nothrow) pkv_decode_graph;
  if (!g) return PKV_ERR_INVALID_ARGUMENT;
  g->desc = d;
  g->sizes.assign(sizes, sizes + num_sizes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // capture from the largest size down, as the pages describe
  g->graphs.assign(num_sizes, nullptr);
  g->execs.assign(num_sizes, nullptr);
  for (int32_t i = num_sizes - 1; i >= 0; --i) {
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
      release(g);
      return hip_failed(e);
    }
    const int rc = enqueue_step(d, g->sizes[i], s);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(s, &graph);
    if (rc != PKV_OK || e != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      release(g);
      return rc != PKV_OK ? rc : hip_failed(e);
    }
    g->graphs[i] = graph;
    e = hipGraphInstantiate(&g->execs[i], graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      release(g);
      return hip_failed(e);
    }
  }
  *out = g;
  return PKV_OK;
}

int pkv_decode_graph_replay(pkv_decode_graph* g, int32_t num_reqs, int32_t num_alloc, int32_t* graph_size,
                            void* stream) {
  if (!g || num_reqs <= 0 || num_alloc < 0 || num_alloc > num_reqs) return PKV_ERR_INVALID_ARGUMENT;
  auto it = std::lower_bound(g->sizes.begin(), g->sizes.end(), num_reqs);
  if (it == g->sizes.end()) return PKV_ERR_INVALID_ARGUMENT;  // larger than the largest captured size
  const size_t k = (size_t)(it - g->sizes.begin());
  const int32_t bs = *it;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const pkv_decode_graph_desc& d = g->desc;
  if (bs > num_reqs) {
    const int32_t pad = bs - num_reqs;
    hipLaunchKernelGGL(pad_kernel, dim3((unsigned)((pad + 255) / 256)), dim3(256), 0, s, d.table_idx, d.cached_len,
                       d.device_len, d.alloc_rows, num_reqs, bs, num_alloc, d.dummy_table_row);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_failed(e);
  }
  hipError_t e = hipGraphLaunch(g->execs[k], s);
  if (e != hipSuccess) return hip_failed(e);
  if (graph_size) *graph_size = bs;
  return PKV_OK;
}

int pkv_decode_graph_destroy(pkv_decode_graph* g) {
  if (!g) return PKV_ERR_INVALID_ARGUMENT;
  release(g);
  return PKV_OK;
}

}  // extern "C"
