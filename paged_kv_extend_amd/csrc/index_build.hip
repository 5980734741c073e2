// Unified KV index build (page "extend_attention.py": build_unified_kv_indices
// and _copy_unified_indices_kernel): per-sequence prefix lengths, the
// running-sum indptr of prefix + new lengths, and the per-sequence
// concatenation of prefix slots and new-token slots -- in one launch.
//
// Grid (bs, ways): workgroup (b, w) finds sequence b's output offset itself,
// U_b = (prefix_kv_indptr[b] - prefix_kv_indptr[0]) + sum_{j<b} extend_seq_lens[j],
// with a cooperative reduction over the lengths (no separate scan launch and
// no host round trip), then copies every ways-th 64-lane run of the segment
// with 8-byte lane loads and stores.  Workgroup (b, 0) writes the indptr
// entry and prefix length of b.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void index_build_kernel(
    const int32_t* __restrict__ prefix_kv_indptr, const int64_t* __restrict__ prefix_kv_indices,
    const int32_t* __restrict__ extend_start_loc, const int32_t* __restrict__ extend_seq_lens,
    const int64_t* __restrict__ extend_kv_indices, int32_t bs, int32_t* __restrict__ unified_kv_indptr,
    int64_t* __restrict__ unified_kv_indices, int32_t* __restrict__ prefix_lens) {
  __shared__ int32_t red[kThreads / 64];
  const int b = blockIdx.x, w = blockIdx.y, ways = gridDim.y, tid = threadIdx.x;
  if (b == 0 && w == 0 && tid == 0) unified_kv_indptr[0] = 0;
  if (b >= bs) return;

  int32_t part = 0;
  for (int j = tid; j < b; j += kThreads) part += extend_seq_lens[j];
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  int32_t ext_before = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) ext_before += red[i];

  const int32_t p_start = prefix_kv_indptr[b];
  const int32_t p_len = prefix_kv_indptr[b + 1] - p_start;
  const int32_t e_start = extend_start_loc[b];
  const int32_t e_len = extend_seq_lens[b];
  const int64_t u = (int64_t)(p_start - prefix_kv_indptr[0]) + ext_before;
  if (w == 0 && tid == 0) {
    unified_kv_indptr[b + 1] = (int32_t)(u + p_len + e_len);
    if (prefix_lens) prefix_lens[b] = p_len;
  }

  // copy in 64-entry runs; run k of the segment goes to workgroup k % ways
  const int lane = tid & 63, wave = tid >> 6;
  const int total = p_len + e_len;
  for (int run = w * (kThreads / 64) + wave; run * 64 < total; run += ways * (kThreads / 64)) {
    const int o = run * 64 + lane;
    if (o < p_len)
      unified_kv_indices[u + o] = prefix_kv_indices[p_start + o];
    else if (o < total)
      unified_kv_indices[u + o] = extend_kv_indices[e_start + (o - p_len)];
  }
}

}  // namespace

hipError_t launch_index_build(const int32_t* prefix_kv_indptr, const int64_t* prefix_kv_indices,
                              const int32_t* extend_start_loc, const int32_t* extend_seq_lens,
                              const int64_t* extend_kv_indices, int32_t bs,
                              int32_t* unified_kv_indptr, int64_t* unified_kv_indices,
                              int32_t* prefix_lens, hipStream_t s) {
  // spread small batches over more workgroups so long segments copy in
  // parallel (a wave's runs are serial round trips: with four sequences of
  // 16 K indices each, 64 ways leave about one run per wave)
  const int ways = bs >= 256 ? 1 : bs >= 32 ? 4 : bs >= 8 ? 16 : 64;
  dim3 grid(bs > 0 ? bs : 1, bs > 0 ? ways : 1);
  hipLaunchKernelGGL(index_build_kernel, grid, dim3(kThreads), 0, s, prefix_kv_indptr,
                     prefix_kv_indices, extend_start_loc, extend_seq_lens, extend_kv_indices, bs,
                     unified_kv_indptr, unified_kv_indices, prefix_lens);
  return hipGetLastError();
}

}  // namespace pkv
