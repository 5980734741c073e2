// The two steps before extend attention (page "flashinfer_backend.py"):
//  * store_kv: the KV-cache store of the new tokens (forward_extend calls
//    set_kv_buffer(layer, cache_loc, k, v) before the paged part reads the
//    pool): K row (t, g) -> pool slot out_cache_loc[t], V likewise.
//  * gather_indices: the prefix indices of a batch from the request-to-token
//    table (create_flashinfer_kv_indices_triton, with the running-sum indptr
//    of call_begin_forward computed here instead of on the host).
// Both are pure data movement, bound by HBM bandwidth.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// One thread moves 16 bytes; consecutive threads take consecutive 16-byte
// chunks of a row (K chunks, then V chunks), so a wave reads and writes whole
// rows.  Chunk i of the launch: row = i / per_row = t * hkv + g.
__global__ __launch_bounds__(kThreads) void store_kv_kernel(StoreArgs a) {
  const uint32_t per_row = a.ck + a.cv;
  const uint32_t total = a.rows * per_row;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads) {
    const uint32_t row = i / per_row, c = i - row * per_row;
    const uint32_t t = row / a.hkv, g = row - t * a.hkv;
    const int64_t slot = a.loc[t];
    const char* src;
    char* dst;
    if (c < a.ck) {
      src = a.k_ext + (int64_t)t * a.ke_st + (int64_t)g * a.ke_sh + c * 16;
      dst = a.k_pool + slot * a.kp_ss + (int64_t)g * a.kp_sh + c * 16;
    } else {
      src = a.v_ext + (int64_t)t * a.ve_st + (int64_t)g * a.ve_sh + (c - a.ck) * 16;
      dst = a.v_pool + slot * a.vp_ss + (int64_t)g * a.vp_sh + (c - a.ck) * 16;
    }
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

// Grid (bs, ways): workgroup (b, w) sums the lengths before b itself (as the
// unified index build does), writes kv_indptr[b+1] (w == 0), and copies
// every ways-th 64-entry run of request b's slots, int32 -> int64.
__global__ __launch_bounds__(kThreads) void gather_indices_kernel(GatherArgs a) {
  __shared__ int32_t red[kThreads / 64];
  const int b = blockIdx.x, w = blockIdx.y, ways = gridDim.y, tid = threadIdx.x;
  if (b == 0 && w == 0 && tid == 0) a.kv_indptr[0] = 0;
  if (b >= a.bs) return;
  int32_t part = 0;
  for (int j = tid; j < b; j += kThreads) part += a.kv_lens[j];
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  int64_t before = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) before += red[i];
  const int32_t len = a.kv_lens[b];
  if (w == 0 && tid == 0) a.kv_indptr[b + 1] = (int32_t)(before + len);
  const int32_t* row = a.req_to_token + a.req_pool_indices[b] * a.stride + (a.kv_start_idx ? a.kv_start_idx[b] : 0);
  const int lane = tid & 63, wave = tid >> 6;
  for (int run = w * (kThreads / 64) + wave; run * 64 < len; run += ways * (kThreads / 64)) {
    const int o = run * 64 + lane;
    // writes stay inside the capacity the caller gave, whatever the lengths hold
    if (o < len && before + o < a.capacity) a.kv_indices[before + o] = (int64_t)row[o];
  }
}

}  // namespace

hipError_t launch_store_kv(const StoreArgs& a, hipStream_t s) {
  const uint64_t total = (uint64_t)a.rows * (a.ck + a.cv);
  if (total == 0) return hipSuccess;
  // a few waves of work per thread: 256 CUs x 8 workgroups resident
  const uint64_t blocks = (total + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(blocks < 2048 * 4 ? blocks : 2048 * 4);
  hipLaunchKernelGGL(store_kv_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather_indices(const GatherArgs& a, hipStream_t s) {
  const int ways = a.bs >= 256 ? 1 : (a.bs >= 32 ? 4 : 16);
  dim3 grid(a.bs > 0 ? a.bs : 1, a.bs > 0 ? ways : 1);
  hipLaunchKernelGGL(gather_indices_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
