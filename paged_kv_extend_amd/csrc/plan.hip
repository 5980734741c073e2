// Device-side work planner for extend attention (one workgroup, no host sync).
//
// Items are (sequence b, KV head g, packed-row tile t).  An item's cost is the
// number of KV tiles it must visit: the prefix plus the new tokens up to the
// last token in its rows (keys past the causal diagonal are never visited).
// Items costing more than a chunk limit are split into near-equal KV ranges
// whose partial softmax states are merged afterwards; the limit starts at
// total / (2 * resident workgroups) so no chunk exceeds half an average
// workgroup's share, and grows when the partial-state budget would overflow.
// Chunks are then ordered heaviest first, so the hardware's in-order
// dispatch approximates longest-processing-time-first scheduling.
//
// The pages' own grids launch one program per (sequence, head, query block)
// with every program visiting all keys (page "extend_attention.py",
// extend_attention_fwd_unified); the split + merge follows the ragged /
// paged split of page "flashinfer_backend.py" (forward_extend, merge_state).
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kBuckets = 4096;

struct Shared {
  int32_t scan[kThreads];
  int64_t red[kThreads / 64];
  int32_t bucket[kBuckets];
};

// Exclusive scan of f(i), i in [0, n), written to out[i]; returns the total.
// Each thread owns a contiguous run; one block scan of the run sums.
template <class F>
__device__ int64_t block_scan(int n, F f, int32_t* out, Shared& sh) {
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int32_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += f(i);
  sh.scan[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int32_t v = tid >= off ? sh.scan[tid - off] : 0;
    __syncthreads();
    sh.scan[tid] += v;
    __syncthreads();
  }
  int32_t run = sh.scan[tid] - sum;
  const int64_t total = sh.scan[kThreads - 1];
  for (int i = lo; i < hi; ++i) {
    const int32_t v = f(i);
    out[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

__device__ int64_t block_sum(int64_t v, Shared& sh) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t t = 0;
  for (int w = 0; w < kThreads / 64; ++w) t += sh.red[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(kThreads) void plan_kernel(PlanArgs a) {
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  const int G = a.group, BM = a.bm, BN = a.bn, H = a.num_kv_heads;
  // scratch: seq_base[bs+1] | cost | chunk_base | part_base | merge_idx | b | g | t  (items)
  int32_t* seq_base = a.scratch;
  int32_t* cost_of = seq_base + a.bs + 1;
  int32_t* chunk_base = cost_of + a.max_items;
  int32_t* part_base = chunk_base + a.max_items;
  int32_t* merge_idx = part_base + a.max_items;
  int32_t* item_b = merge_idx + a.max_items;
  int32_t* item_g = item_b + a.max_items;
  int32_t* item_t = item_g + a.max_items;

  // 1. items per sequence: H * ceil(E_b * G / BM)
  auto seq_items = [&](int b) {
    const int E = a.qo_indptr[b + 1] - a.qo_indptr[b];
    return H * ceil_div(E * G, BM);
  };
  const int n_items = (int)block_scan(a.bs, seq_items, seq_base, sh);
  if (tid == 0) seq_base[a.bs] = n_items;
  __syncthreads();

  // 2. cost of every item in KV tiles; items ordered (b, g, t)
  int64_t my_total = 0;
  for (int n = tid; n < n_items; n += kThreads) {
    int lo = 0, hi = a.bs - 1;  // last b with seq_base[b] <= n
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seq_base[mid] <= n) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int E = a.qo_indptr[b + 1] - a.qo_indptr[b];
    const int P = a.kv_indptr[b + 1] - a.kv_indptr[b];
    const int T = ceil_div(E * G, BM);
    const int t = (n - seq_base[b]) % T;
    const int row_hi = min((t + 1) * BM, E * G) - 1;
    const int cost = ceil_div(P + row_hi / G + 1, BN);
    cost_of[n] = cost;
    item_b[n] = b;
    item_g[n] = (n - seq_base[b]) / T;
    item_t[n] = t;
    my_total += cost;
  }
  const int64_t total = block_sum(my_total, sh);

  // 3. chunk limit: half an average share per resident workgroup, grown until
  //    the split chunks fit the partial-state budget
  int64_t chunk = (total + 2 * (int64_t)a.slots - 1) / (2 * (int64_t)a.slots);
  if (chunk < a.min_chunk) chunk = a.min_chunk;
  for (;;) {
    int64_t parts = 0;
    for (int n = tid; n < n_items; n += kThreads) {
      const int c = cost_of[n];
      if (c > chunk) parts += (c + chunk - 1) / chunk;
    }
    parts = block_sum(parts, sh);
    if (parts <= a.part_budget) break;
    chunk *= 2;
  }
  auto nsplit = [&](int n) {
    const int c = cost_of[n];
    return c > chunk ? (int)((c + chunk - 1) / chunk) : 1;
  };

  // 4. per-item offsets of partial slots and merge records
  const int n_work = (int)block_scan(n_items, nsplit, chunk_base, sh);
  block_scan(n_items, [&](int n) { int k = nsplit(n); return k > 1 ? k : 0; }, part_base, sh);
  const int n_merge = (int)block_scan(n_items, [&](int n) { return nsplit(n) > 1 ? 1 : 0; }, merge_idx, sh);

  // 5. heaviest first: counting sort of chunks by size (descending); the order
  //    among equal sizes only affects scheduling, never the results
  for (int i = tid; i < kBuckets; i += kThreads) sh.bucket[i] = 0;
  __syncthreads();
  for (int n = tid; n < n_items; n += kThreads) {
    const int c = cost_of[n], k = nsplit(n);
    for (int s = 0; s < k; ++s) {
      const int sz = (int)((int64_t)c * (s + 1) / k - (int64_t)c * s / k);
      atomicAdd(&sh.bucket[min(sz, kBuckets - 1)], 1);
    }
  }
  __syncthreads();
  if (tid == 0) {  // descending exclusive scan over bucket counts
    int run = 0;
    for (int i = kBuckets - 1; i >= 0; --i) {
      const int v = sh.bucket[i];
      sh.bucket[i] = run;
      run += v;
    }
  }
  __syncthreads();
  for (int n = tid; n < n_items; n += kThreads) {
    const int c = cost_of[n], k = nsplit(n);
    for (int s = 0; s < k; ++s) {
      const int k0 = (int)((int64_t)c * s / k), k1 = (int)((int64_t)c * (s + 1) / k);
      const int pos = atomicAdd(&sh.bucket[min(k1 - k0, kBuckets - 1)], 1);
      WorkItem w;
      w.b = item_b[n];
      w.g = item_g[n];
      w.t = item_t[n];
      w.kt_begin = k0;
      w.kt_end = k1;
      w.part = k > 1 ? part_base[n] + s : -1;
      w.pad0 = 0;
      w.pad1 = 0;
      a.work[pos] = w;
    }
    if (k > 1) {
      MergeItem m;
      m.b = item_b[n];
      m.g = item_g[n];
      m.t = item_t[n];
      m.part_base = part_base[n];
      m.n = k;
      m.pad0 = m.pad1 = m.pad2 = 0;
      a.merge[merge_idx[n]] = m;
    }
  }
  if (tid == 0) {
    a.hdr->num_work = n_work;
    a.hdr->num_merge = n_merge;
    a.hdr->chunk_tiles = (int32_t)chunk;
    a.hdr->total_tiles = (int32_t)total;
    a.hdr->num_items = n_items;
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
