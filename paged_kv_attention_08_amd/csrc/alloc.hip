// Page allocator on the GPU: a ring of free page-start rows that
// build_attn_metadata's alloc_rows input is taken from, so a step's
// allocation needs no host round trip (and can sit in a captured graph).
//
// mini-sglang learning notes, page-table passage: the scheduler counts, page
// aligned, the new pages each request needs over [cached_len, device_len),
// takes them from free_slots in one batch and writes the page table; the free
// list is kept page aligned.  Deep dive section 3.6: freed entries are
// appended to the free list.
//
// The batch's pages are the next n entries of the ring, request by request in
// batch order (build_attn_metadata's running count of new pages gives each
// request its offset), so allocation is a count followed by one contiguous
// ring copy; freeing appends at the tail.  One workgroup per call: the work is
// a few thousand integers.
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kThreads = 1024;

__device__ inline int32_t pages_for(int32_t c, int32_t d, int32_t s) {
  if (c < 0 || c > d) return 0;  // invalid lengths need no page (build_attn_metadata counts the same way)
  return (d + s - 1) / s - (c + s - 1) / s;
}

__device__ inline long long block_sum(long long v, long long* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  long long tot = 0;
  for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
  __syncthreads();
  return tot;
}

__global__ void __launch_bounds__(kThreads) alloc_pages_kernel(AllocArgs a) {
  __shared__ long long red[kThreads / 64];
  const int32_t head = a.state[0];
  const int32_t count = a.state[1];
  long long need = 0;
  for (int i = threadIdx.x; i < a.B; i += kThreads) need += pages_for(a.cached_len[i], a.device_len[i], a.page_size);
  need = block_sum(need, red);
  if (need > count || need > a.max_alloc || head < 0 || head >= a.capacity || count < 0 || count > a.capacity) {
    // nothing is taken; the entries the batch would read become -1 so that
    // build_attn_metadata maps none of its new tokens
    const long long n = need < a.max_alloc ? need : a.max_alloc;
    for (long long j = threadIdx.x; j < n; j += kThreads) a.alloc_rows[j] = -1;
    if (threadIdx.x == 0) raise_status(a.status, PKV_STATUS_OUT_OF_PAGES);
    return;
  }
  int bad = 0;
#pragma unroll 4
  for (long long j = threadIdx.x; j < need; j += kThreads) {
    long long idx = head + j;
    if (idx >= a.capacity) idx -= a.capacity;
    const int32_t row = a.rows[idx];
    if (row < 0 || row % a.page_size != 0 || row >= a.num_pool_rows) bad = 1;
    a.alloc_rows[j] = row;  // a bad row is passed on; build_attn_metadata reports and skips its tokens
  }
  if (bad) raise_status(a.status, PKV_STATUS_BAD_ALLOC);
  __syncthreads();  // every thread has read state
  if (threadIdx.x == 0) {
    long long h = head + need;
    if (h >= a.capacity) h -= a.capacity;
    a.state[0] = (int32_t)h;
    a.state[1] = count - (int32_t)need;
  }
}

__global__ void __launch_bounds__(kThreads) free_pages_kernel(AllocArgs a) {
  __shared__ long long red[kThreads / 64];
  const int32_t head = a.state[0];
  const int32_t count = a.state[1];
  long long bad = 0;
  for (int j = threadIdx.x; j < a.num_free; j += kThreads) {
    const int32_t row = a.free_rows[j];
    bad += (row < 0 || row % a.page_size != 0 || row >= a.num_pool_rows);
  }
  bad = block_sum(bad, red);
  if (bad || head < 0 || head >= a.capacity || count < 0 || (long long)count + a.num_free > a.capacity) {
    if (threadIdx.x == 0) raise_status(a.status, bad ? PKV_STATUS_BAD_ALLOC : PKV_STATUS_FREE_OVERFLOW);
    return;  // nothing freed
  }
#pragma unroll 4
  for (int j = threadIdx.x; j < a.num_free; j += kThreads) {
    long long idx = (long long)head + count + j;
    if (idx >= a.capacity) idx -= a.capacity;
    if (idx >= a.capacity) idx -= a.capacity;
    a.rows[idx] = a.free_rows[j];
  }
  __syncthreads();
  if (threadIdx.x == 0) a.state[1] = count + a.num_free;
}

__global__ void free_list_reset_kernel(int32_t* state, int32_t num_free) {
  if (threadIdx.x == 0) {
    state[0] = 0;
    state[1] = num_free;
  }
}

}  // namespace

hipError_t launch_alloc_pages(const AllocArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(alloc_pages_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_free_pages(const AllocArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(free_pages_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_free_list_reset(int32_t* state, int32_t num_free, hipStream_t s) {
  hipLaunchKernelGGL(free_list_reset_kernel, dim3(1), dim3(64), 0, s, state, num_free);
  return hipGetLastError();
}

}  // namespace pkv
