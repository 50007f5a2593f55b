// kv_store: scatter of the batch's new K/V rows into the pool at out_loc.
//
// mini-sglang learning notes, store_kv passage: at every layer the attention
// backend first writes the freshly computed K/V of the batch to the pool
// rows named by out_loc (raw physical positions).  The pages' kernel gives one
// warp per token row; here a token row (Hkv * d * 2 bytes, 2 KiB at 8 KV heads)
// is moved as 16-byte vectors, with consecutive lanes on consecutive vectors
// of the same row so that every wavefront reads and writes whole contiguous
// 1 KiB runs.  The work is pure HBM traffic: 2 reads + 2 writes of a row per
// token plus the 4-byte out_loc entry.
#include "kernels.hpp"

namespace pkv {

__global__ void __launch_bounds__(256) kv_store_kernel(StoreArgs a) {
  const int64_t total = a.num_tokens * a.row_vec;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t t = idx / a.row_vec;
    const int32_t c = (int32_t)(idx - t * a.row_vec);
    int32_t row = a.out_loc[t];
    // the source vectors do not depend on the row: their loads go out with
    // the out_loc load, so a thread waits for one memory round trip, not two
    const int64_t src = t * a.row_vec + c;
    uint4 kv = a.k_new[src];
    uint4 vv = a.v_new[src];
    // keeps the loads above the branch (the compiler would sink them into it)
    asm volatile("" : "+v"(row), "+v"(kv.x), "+v"(kv.y), "+v"(kv.z), "+v"(kv.w), "+v"(vv.x), "+v"(vv.y), "+v"(vv.z),
                 "+v"(vv.w));
    if (row < 0 || (int64_t)row >= a.num_rows) {
      // -1 marks a token build_attn_metadata could not map (already reported)
      if (c == 0 && row != -1) raise_status(a.status, PKV_STATUS_BAD_OUT_LOC);
      continue;
    }
    const int64_t dst = (int64_t)row * a.row_stride_vec + c;
    a.k_pool[dst] = kv;
    a.v_pool[dst] = vv;
  }
}

hipError_t launch_kv_store(const StoreArgs& a, hipStream_t s) {
  const int64_t total = a.num_tokens * a.row_vec;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
