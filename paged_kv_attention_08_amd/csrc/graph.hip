// pkv_decode_graph_*: the decode step (build_attn_metadata_store ->
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
// real requests into the fixed buffers and the number of real requests into
// the graph's first kernel node (its argument block), and the graph's first
// kernel turns the remaining slots into dummy requests before planning.
#include <algorithm>
#include <new>
#include <vector>

#include "kernels.hpp"

struct pkv_decode_graph {
  pkv_decode_graph_desc desc;
  std::vector<int32_t> sizes;          // ascending
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
  std::vector<hipGraphNode_t> plan_nodes;   // the metadata plan kernel of each graph (its only root)
  std::vector<pkv::MetaArgs> plan_args;     // that node's argument block as captured
  std::vector<int32_t> plan_pad_from;       // the real-request count the node's arguments now hold
};

using namespace pkv;

namespace {

// The step on a batch of bs decode requests, enqueued on s (captured by the
// caller): build_attn_metadata_store, then paged_decode_attn.  *plan_args
// receives the metadata plan kernel's argument block.
int enqueue_step(const pkv_decode_graph_desc& d, int32_t bs, MetaArgs* plan_args, hipStream_t s) {
  pkv_batch b;
  b.num_reqs = bs;
  b.num_decode = bs;
  b.num_tokens = bs;
  b.table_idx = d.table_idx;
  b.cached_len = d.cached_len;
  b.device_len = d.device_len;
  MetaArgs a;
  StoreArgs st;
  int rc = prepare_metadata_store(&b, &d.page_table, &d.pool, d.alloc_rows, bs, d.num_qo_heads, &d.meta, d.k_new,
                                  d.v_new, &a, &st);
  if (rc != PKV_OK) return rc;
  // padding: set per replay in the plan node's arguments (none at capture)
  a.pad_from = bs;
  a.dummy_row = d.dummy_table_row;
  a.pad_table_idx = d.table_idx;
  a.pad_cached_len = d.cached_len;
  a.pad_device_len = d.device_len;
  a.pad_alloc_rows = d.alloc_rows;
  *plan_args = a;
  // metadata and store (one kernel for up to 1024 requests), then attention
  hipError_t e = launch_metadata_store(a, st, s);
  if (e != hipSuccess) return hip_failed(e);
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

// The graph's root: the metadata plan kernel, launched first in the capture.
hipError_t find_plan_node(hipGraph_t graph, hipGraphNode_t* node) {
  size_t n = 0;
  hipError_t e = hipGraphGetRootNodes(graph, nullptr, &n);
  if (e != hipSuccess) return e;
  if (n != 1) return hipErrorInvalidValue;
  e = hipGraphGetRootNodes(graph, node, &n);
  if (e != hipSuccess) return e;
  hipGraphNodeType type;
  e = hipGraphNodeGetType(*node, &type);
  if (e != hipSuccess) return e;
  return type == hipGraphNodeTypeKernel ? hipSuccess : hipErrorInvalidValue;
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
  if (!g) return PKV_ERR_HOST_ALLOC;
  try {
    g->desc = d;
    g->sizes.assign(sizes, sizes + num_sizes);
    g->graphs.assign(num_sizes, nullptr);
    g->execs.assign(num_sizes, nullptr);
    g->plan_nodes.assign(num_sizes, nullptr);
    g->plan_args.resize(num_sizes);
    g->plan_pad_from.assign(num_sizes, -1);
  } catch (const std::bad_alloc&) {
    delete g;
    return PKV_ERR_HOST_ALLOC;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // capture from the largest size down, as the pages describe
  for (int32_t i = num_sizes - 1; i >= 0; --i) {
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
      release(g);
      return hip_failed(e);
    }
    const int rc = enqueue_step(d, g->sizes[i], &g->plan_args[i], s);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(s, &graph);
    if (rc != PKV_OK || e != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      release(g);
      return rc != PKV_OK ? rc : hip_failed(e);
    }
    g->graphs[i] = graph;
    e = find_plan_node(graph, &g->plan_nodes[i]);
    if (e == hipSuccess) e = hipGraphInstantiate(&g->execs[i], graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      release(g);
      return hip_failed(e);
    }
  }
  *out = g;
  return PKV_OK;
}

int pkv_decode_graph_replay(pkv_decode_graph* g, int32_t num_reqs, int32_t* graph_size, void* stream) {
  if (!g || num_reqs <= 0) return PKV_ERR_INVALID_ARGUMENT;
  auto it = std::lower_bound(g->sizes.begin(), g->sizes.end(), num_reqs);
  if (it == g->sizes.end()) return PKV_ERR_INVALID_ARGUMENT;  // larger than the largest captured size
  const size_t k = (size_t)(it - g->sizes.begin());
  hipStream_t s = static_cast<hipStream_t>(stream);
  // slots [num_reqs, bs) become dummy requests inside the graph's plan kernel;
  // its arguments are rewritten only when the count differs from the one they
  // hold (a decode loop mostly replays one size with one count)
  hipError_t e = hipSuccess;
  if (g->plan_pad_from[k] != num_reqs) {
    MetaArgs a = g->plan_args[k];
    a.pad_from = num_reqs;
    MetaArgs node_args;
    void* argv[1];
    hipKernelNodeParams p;
    metadata_plan_node(a, &node_args, argv, &p);
    e = hipGraphExecKernelNodeSetParams(g->execs[k], g->plan_nodes[k], &p);
    if (e != hipSuccess) {
      g->plan_pad_from[k] = -1;
      return hip_failed(e);
    }
    g->plan_pad_from[k] = num_reqs;
  }
  e = hipGraphLaunch(g->execs[k], s);
  if (e != hipSuccess) return hip_failed(e);
  if (graph_size) *graph_size = *it;
  return PKV_OK;
}

int pkv_decode_graph_destroy(pkv_decode_graph* g) {
  if (!g) return PKV_ERR_INVALID_ARGUMENT;
  release(g);
  return PKV_OK;
}

}  // extern "C"
