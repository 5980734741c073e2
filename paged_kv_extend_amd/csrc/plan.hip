// Device-side work planner for extend attention (one workgroup, no host sync).
//
// Items are (sequence b, KV head g, packed-row tile t).  An item's cost is the
// number of KV tiles it must visit: the prefix plus the new tokens up to the
// last token in its rows (keys past the causal diagonal are never visited).
// An item costing more than one resident workgroup's average share (total
// cost / resident workgroups) is split into near-equal KV ranges whose
// partial softmax states are merged afterwards; the limit grows when the
// partial-state budget would overflow.
//
// Placement: workgroup i of a launch runs on XCD i mod 8, and each XCD has
// its own L2.  The (b, g, t, chunk)-ordered cost sequence is cut into one
// contiguous, equal-cost range per XCD (a chunk goes to the range holding its
// midpoint), so the q-tiles of one (sequence, KV head) -- which read the same
// prefix K/V -- share an L2 while every XCD gets the same work.  Within an
// XCD chunks run heaviest first (counting sort over 256 size classes), which
// with in-order dispatch approximates longest-processing-time-first; slot
// rank*8 + xcd holds the XCD's rank-th chunk and unused slots hold empty items.
//
// The pages' own grids launch one program per (sequence, head, query block)
// with every program visiting all keys (page "extend_attention.py",
// extend_attention_fwd_unified); the split + merge follows the ragged /
// paged split of page "flashinfer_backend.py" (forward_extend, merge_state).
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBuckets = 256;
constexpr int kMaxXcd = 8;
constexpr int kSeqLds = 8192;  // sequence offsets kept in LDS up to this batch size

struct Shared {
  int32_t wave_tot[kWaves];
  int32_t wave_tot3[kWaves][3];
  int64_t red[kWaves];
  int32_t bucket[kMaxXcd * kBuckets];
  int32_t bin_count[kMaxXcd];
  int32_t bin_start[kMaxXcd];
  int32_t seq_base[kSeqLds + 1];
};

// Exclusive block-wide scan of one int per thread; returns the block total.
__device__ int32_t block_excl_scan(int32_t v, int32_t* total, Shared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(inc, off);
    if (lane >= off) inc += u;
  }
  if (lane == 63) sh.wave_tot[w] = inc;
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int32_t t = sh.wave_tot[i];
    before += i < w ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Exclusive block-wide scans of three ints per thread in one pass.
__device__ int3 block_excl_scan3(int3 v, int3* total, Shared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int3 inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ux = __shfl_up(inc.x, off), uy = __shfl_up(inc.y, off), uz = __shfl_up(inc.z, off);
    if (lane >= off) {
      inc.x += ux;
      inc.y += uy;
      inc.z += uz;
    }
  }
  if (lane == 63) {
    sh.wave_tot3[w][0] = inc.x;
    sh.wave_tot3[w][1] = inc.y;
    sh.wave_tot3[w][2] = inc.z;
  }
  __syncthreads();
  int3 before = make_int3(0, 0, 0), all = make_int3(0, 0, 0);
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int tx = sh.wave_tot3[i][0], ty = sh.wave_tot3[i][1], tz = sh.wave_tot3[i][2];
    if (i < w) {
      before.x += tx;
      before.y += ty;
      before.z += tz;
    }
    all.x += tx;
    all.y += ty;
    all.z += tz;
  }
  __syncthreads();
  *total = all;
  return make_int3(before.x + inc.x - v.x, before.y + inc.y - v.y, before.z + inc.z - v.z);
}

__device__ int64_t block_sum(int64_t v, Shared& sh) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += sh.red[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(kThreads) void plan_kernel(PlanArgs a) {
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  const int G = a.group, BM = a.bm, BN = a.bn, H = a.num_kv_heads;
  // global scratch: seq_base[bs+1] | cost | part_base | merge_idx | b | g | t | cum  (per item)
  int32_t* seq_base_g = a.scratch;
  int32_t* cost_of = seq_base_g + a.bs + 1;
  int32_t* part_base = cost_of + a.max_items;
  int32_t* merge_idx = part_base + a.max_items;
  int32_t* item_b = merge_idx + a.max_items;
  int32_t* item_g = item_b + a.max_items;
  int32_t* item_t = item_g + a.max_items;
  int32_t* cum_cost = item_t + a.max_items;  // exclusive running sum of item costs
  const bool seq_in_lds = a.bs <= kSeqLds;
  int32_t* seq_base = seq_in_lds ? sh.seq_base : seq_base_g;

  // zero row read for keys past a sequence
  for (int i = tid; i < kZeroRowBytes / 16; i += kThreads)
    reinterpret_cast<uint4*>(a.zero_row)[i] = make_uint4(0, 0, 0, 0);

  // 1. items per sequence, H * ceil(E_b G / BM); exclusive scan in runs of kThreads
  int32_t carry = 0;
  for (int base = 0; base < a.bs; base += kThreads) {
    const int b = base + tid;
    int32_t v = 0;
    if (b < a.bs) v = H * ceil_div((a.qo_indptr[b + 1] - a.qo_indptr[b]) * G, BM);
    int32_t tot;
    const int32_t ex = block_excl_scan(v, &tot, sh);
    if (b < a.bs) seq_base[b] = carry + ex;
    carry += tot;
  }
  const int n_items = carry;
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
    const int local = n - seq_base[b];
    const int t = local % T;
    const int row_hi = min((t + 1) * BM, E * G) - 1;
    const int cost = ceil_div(P + row_hi / G + 1, BN);
    cost_of[n] = cost;
    item_b[n] = b;
    item_g[n] = local / T;
    item_t[n] = t;
    my_total += cost;
  }
  const int64_t total = block_sum(my_total, sh);

  // 3. chunk limit: one average share per resident workgroup, grown until the
  //    split chunks fit the partial-state budget
  int64_t chunk = (total + a.slots - 1) / a.slots;
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

  // 4. partial-slot and merge-record offsets of split items, running cost (scans in runs)
  int32_t pcarry = 0, mcarry = 0, ccarry = 0;
  for (int base = 0; base < n_items; base += kThreads) {
    const int n = base + tid;
    int k = 1, c = 0;
    if (n < n_items) {
      c = cost_of[n];
      k = c > chunk ? (int)((c + chunk - 1) / chunk) : 1;
    }
    int3 tot;
    const int3 ex = block_excl_scan3(make_int3(k > 1 ? k : 0, k > 1 ? 1 : 0, c), &tot, sh);
    if (n < n_items) {
      part_base[n] = pcarry + ex.x;
      merge_idx[n] = mcarry + ex.y;
      cum_cost[n] = ccarry + ex.z;
    }
    const int32_t ptot = tot.x, mtot = tot.y, ctot = tot.z;
    pcarry += ptot;
    mcarry += mtot;
    ccarry += ctot;
  }

  // 5. XCD bin of every chunk (midpoint rule), then heaviest first inside a bin
  const int64_t cls_div = (chunk + kBuckets - 1) / kBuckets;  // chunk sizes are <= chunk
  auto size_class = [&](int sz) { return (int)min<int64_t>(kBuckets - 1, (sz - 1) / cls_div); };
  int X = a.xcds < 1 ? 1 : (a.xcds > kMaxXcd ? kMaxXcd : a.xcds);
  auto bin_of = [&](int n, int k0, int k1) {
    const int64_t mid2 = 2 * (int64_t)cum_cost[n] + k0 + k1;  // twice the chunk midpoint
    return (int)min<int64_t>(X - 1, mid2 * X / (2 * (total > 0 ? total : 1)));
  };
  int32_t my_chunks = 0;
  int max_count = 0;
  for (int attempt = 0; attempt < 2; ++attempt) {
    for (int i = tid; i < kMaxXcd * kBuckets; i += kThreads) sh.bucket[i] = 0;
    __syncthreads();
    my_chunks = 0;
    for (int n = tid; n < n_items; n += kThreads) {
      const int c = cost_of[n];
      const int k = c > chunk ? (int)((c + chunk - 1) / chunk) : 1;
      my_chunks += k;
      for (int s = 0; s < k; ++s) {
        const int k0 = (int)((int64_t)c * s / k), k1 = (int)((int64_t)c * (s + 1) / k);
        atomicAdd(&sh.bucket[bin_of(n, k0, k1) * kBuckets + (kBuckets - 1 - size_class(k1 - k0))], 1);
      }
    }
    __syncthreads();
    // one exclusive scan over all (bin, class) counters, two per thread; a bin's
    // ranks are offsets from its first counter's scan value
    {
      const int i0 = 2 * tid;
      const int32_t v0 = i0 < X * kBuckets ? sh.bucket[i0] : 0;
      const int32_t v1 = i0 + 1 < X * kBuckets ? sh.bucket[i0 + 1] : 0;
      int32_t tot;
      const int32_t ex = block_excl_scan(v0 + v1, &tot, sh);
      if (i0 < X * kBuckets) sh.bucket[i0] = ex;
      if (i0 + 1 < X * kBuckets) sh.bucket[i0 + 1] = ex + v0;
      __syncthreads();
      if (tid < X) {
        sh.bin_start[tid] = sh.bucket[tid * kBuckets];
        sh.bin_count[tid] = (tid + 1 < X ? sh.bucket[(tid + 1) * kBuckets] : tot) - sh.bucket[tid * kBuckets];
      }
      __syncthreads();
    }
    max_count = 0;
    for (int x = 0; x < X; ++x) max_count = max(max_count, sh.bin_count[x]);
    if ((int64_t)max_count * X <= a.max_work || X == 1) break;
    X = 1;  // bins too uneven for the grid: plain heaviest-first order
    __syncthreads();
  }
  for (int n = tid; n < n_items; n += kThreads) {
    const int c = cost_of[n];
    const int k = c > chunk ? (int)((c + chunk - 1) / chunk) : 1;
    const int b = item_b[n], ig = item_g[n], itt = item_t[n];
    for (int s = 0; s < k; ++s) {
      const int k0 = (int)((int64_t)c * s / k), k1 = (int)((int64_t)c * (s + 1) / k);
      const int x = bin_of(n, k0, k1);
      const int rank = atomicAdd(&sh.bucket[x * kBuckets + (kBuckets - 1 - size_class(k1 - k0))], 1) -
                       sh.bin_start[x];
      WorkItem w;
      w.b = b;
      w.g = ig;
      w.t = itt;
      w.kt_begin = k0;
      w.kt_end = k1;
      w.part = k > 1 ? part_base[n] + s : -1;
      w.pad0 = 0;
      w.pad1 = 0;
      a.work[rank * X + x] = w;
    }
    if (k > 1) {
      MergeItem m;
      m.b = b;
      m.g = ig;
      m.t = itt;
      m.part_base = part_base[n];
      m.n = k;
      m.pad0 = m.pad1 = m.pad2 = 0;
      a.merge[merge_idx[n]] = m;
    }
  }
  // unused slots of shorter bins hold empty items
  for (int x = 0; x < X; ++x) {
    for (int rank = sh.bin_count[x] + tid; rank < max_count; rank += kThreads) {
      WorkItem w;
      w.b = -1;
      w.g = w.t = w.kt_begin = w.kt_end = 0;
      w.part = -1;
      w.pad0 = w.pad1 = 0;
      a.work[rank * X + x] = w;
    }
  }
  const int64_t n_chunks = block_sum(my_chunks, sh);
  if (tid == 0) {
    a.hdr->num_work = max_count * X;  // grid slots in use, empty items included
    a.hdr->num_chunks = (int32_t)n_chunks;
    a.hdr->xcds = X;
    a.hdr->num_merge = mcarry;
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
