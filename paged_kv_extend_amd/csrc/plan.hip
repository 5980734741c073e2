// Device-side work planner for extend attention (one workgroup, no host sync).
//
// Items are (sequence b, KV head g, packed-row tile t).  An item's cost is the
// number of KV tiles it must visit: the prefix plus the new tokens up to the
// last token in its rows (keys past the causal diagonal are never visited).
// An item costing more than one resident workgroup's average share (total
// cost / resident workgroups) is split into KV ranges of that many tiles (the
// remainder last) whose partial softmax states are merged afterwards; the
// limit grows when the partial-state budget would overflow.  Every work
// record also carries its sequence's key bounds, so that a workgroup's first
// loads depend on the record alone.
//
// Placement: workgroup i of a launch runs on XCD i mod 8, and each XCD has
// its own L2.  With fewer than three chunks per resident workgroup, the
// (b, g, t, chunk)-ordered cost sequence is cut into one contiguous,
// equal-cost range per XCD (a chunk goes to the range holding its midpoint),
// so the q-tiles of one (sequence, KV head) -- which read the same prefix
// K/V -- share an L2 while every XCD gets the same work.  Within an XCD
// chunks run heaviest first (counting sort over 256 size classes), which
// with in-order dispatch approximates longest-processing-time-first; slot
// rank*8 + xcd holds the XCD's rank-th chunk and unused slots hold empty
// items.  With more chunks per workgroup, one heaviest-first list over all
// slots balances the CUs better than the ranges keep L2 sharing.
//
// The pages' own grids launch one program per (sequence, head, query block)
// with every program visiting all keys (page "extend_attention.py",
// extend_attention_fwd_unified); the split + merge follows the ragged /
// paged split of page "flashinfer_backend.py" (forward_extend, merge_state).
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBuckets = 256;
constexpr int kMaxXcd = 8;
constexpr int kSeqLds = 2048;   // per-sequence arrays kept in LDS up to this batch size
constexpr int kItemLds = 8192;  // per-item arrays kept in LDS up to this many items

struct Shared {
  int32_t wave_tot[2][3][kWaves];  // two buffers, used by alternate scans
  int32_t bucket[kMaxXcd * kBuckets];
  int32_t bin_start[kMaxXcd];
  int32_t seq_base[kSeqLds + 1];  // first item of sequence b
  int32_t seq_e[kSeqLds];         // new tokens E_b
  int32_t seq_p[kSeqLds];         // prefix tokens P_b
  int32_t seq_q0[kSeqLds];        // first new-token row qo_indptr[b]
  int32_t seq_kvs[kSeqLds];       // first index kv_indptr[b]
  int32_t seq_span[kSeqLds];      // indices kv_indptr[b + 1] - kv_indptr[b]
  int32_t cum[kItemLds + 1];      // exclusive running sum of the items' KV tiles
  int32_t pm[kItemLds];           // partial base << 16 | merge index (split items)
  int32_t cb[kItemLds + 1];       // first chunk of item n (the item's cost until chunks are cut)
};

// Inclusive scan over the 64 lanes of a wave with DPP: shifts by 1, 2, 4, 8
// inside each row of 16 lanes, then the row totals broadcast to later rows.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive block-wide scans of up to three ints per thread (each value and
// each total must fit 31 bits); returns the scans, sets the totals.  Buffer
// `buf` of the wave totals must alternate between consecutive calls: the
// barrier inside the next call is what orders the reads of this one before
// the writes of the call after it, so no barrier closes a scan.
template <int N>
__device__ void block_excl_scan(const int (&v)[N], int (&ex)[N], int64_t (&total)[N], Shared& sh, int buf) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) inc[i] = wave_incl_scan(v[i]);
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < N; ++i) sh.wave_tot[buf][i][w] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int4 t0 = *reinterpret_cast<const int4*>(&sh.wave_tot[buf][i][0]);
    const int4 t1 = *reinterpret_cast<const int4*>(&sh.wave_tot[buf][i][4]);
    const int t[kWaves] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
    int before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      before += k < w ? t[k] : 0;
      all += t[k];
    }
    ex[i] = before + inc[i] - v[i];
    total[i] = all;
  }
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// n / d for 0 <= n < 2^31 and 0 < d < 2^31, given inv = 1.0 / d: the double
// product lies within 2^-21 of n / d, so its truncation is the quotient or
// one less, and the remainder settles which (a few instructions instead of
// the ~40 of a 32-bit integer divide)
__device__ __forceinline__ int div_by(int n, int d, double inv) {
  int q = (int)((double)n * inv);
  const int r = n - q * d;
  q += r >= d ? 1 : 0;
  q -= r < 0 ? 1 : 0;
  return q;
}

// Per-item arrays in LDS when the batch fits (the only global reads are the
// indptrs), else in the global scratch.  Sequences, items and chunks are
// handed out in contiguous runs per thread, so each pass is a local walk,
// one block scan and a second local walk, whatever the batch size; the walks
// over chunks spread an item cut into many chunks over many threads.
template <bool LDS_ARRAYS>
__device__ void plan_body(const PlanArgs& a, Shared& sh) {
  const int tid = threadIdx.x;
  const int G = a.group, BM = a.bm, BN = a.bn, H = a.num_kv_heads;
  const int lbm = __builtin_ctz(BM), lbn = __builtin_ctz(BN);  // powers of two (launch_plan checks)
  const double inv_g = 1.0 / G;
  int scan_no = 0;  // alternates the scans' buffers (the same sequence of scans on every thread)
  // row tiles of a sequence with E new tokens (E G < 2^31: the host checks)
  auto row_tiles = [&](int E) { return (int)(((uint32_t)(E * G) + (uint32_t)(BM - 1)) >> lbm); };
  // global scratch: seq_base[bs+1] | E | P | q0 | kvs | span (bs each) | cum[items+1] | pm[items] | cb[items+1]
  int32_t* seq_base = LDS_ARRAYS ? sh.seq_base : a.scratch;
  int32_t* seq_e = LDS_ARRAYS ? sh.seq_e : a.scratch + a.bs + 1;
  int32_t* seq_p = LDS_ARRAYS ? sh.seq_p : a.scratch + 2 * a.bs + 1;
  int32_t* seq_q0 = LDS_ARRAYS ? sh.seq_q0 : a.scratch + 3 * a.bs + 1;
  int32_t* seq_kvs = LDS_ARRAYS ? sh.seq_kvs : a.scratch + 4 * a.bs + 1;
  int32_t* seq_span = LDS_ARRAYS ? sh.seq_span : a.scratch + 5 * a.bs + 1;
  int32_t* cum = LDS_ARRAYS ? sh.cum : a.scratch + 6 * a.bs + 1;
  int32_t* pm = LDS_ARRAYS ? sh.pm : cum + a.max_items + 1;
  int32_t* cb = LDS_ARRAYS ? sh.cb : pm + a.max_items;
  // the placement's counters, zeroed here (the barriers of the first scans order it)
  for (int i = tid; i < kMaxXcd * kBuckets; i += kThreads) sh.bucket[i] = 0;

  // 1. per sequence: E, P and items H * ceil(E G / BM), exclusive scan
  const int spt = ceil_div(a.bs, kThreads);  // sequences per thread
  const int s0 = min(a.bs, tid * spt), s1 = min(a.bs, s0 + spt);
  int local = 0;
  for (int b = s0; b < s1; ++b) {
    const int q0 = a.qo_indptr[b], E = a.qo_indptr[b + 1] - q0;
    const int kvs = a.kv_indptr[b], span = a.kv_indptr[b + 1] - kvs;
    // prefix keys: the sequence's index span, or prefix_lens[b] for a unified call
    const int P = a.prefix_lens ? a.prefix_lens[b] : span;
    seq_e[b] = E;
    seq_p[b] = P;
    seq_q0[b] = q0;
    seq_kvs[b] = kvs;
    seq_span[b] = span;
    local += H * row_tiles(E);
  }
  {
    int v[1] = {local}, ex[1];
    int64_t tot[1];
    block_excl_scan<1>(v, ex, tot, sh, scan_no++ & 1);
    int run = ex[0];
    for (int b = s0; b < s1; ++b) {
      seq_base[b] = run;
      run += H * row_tiles(seq_e[b]);
    }
    if (tid == 0) seq_base[a.bs] = (int)tot[0];
    local = (int)tot[0];
  }
  const int n_items = local;
  __syncthreads();
  if (n_items > a.max_items) {
    // qo_indptr holds more rows than the descriptor's total_q_tokens allows:
    // plan nothing (the attention and merge launches then do nothing)
    if (tid == 0) {
      a.hdr->num_work = 0;
      a.hdr->num_merge = 0;
      a.hdr->num_chunks = 0;
      a.hdr->num_items = n_items;
    }
    return;
  }

  // (b, g, t) of item n: items are ordered (b, g, t)
  auto decode = [&](int n, int& b, int& g, int& t) {
    int lo = 0, hi = a.bs - 1;  // last b with seq_base[b] <= n
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seq_base[mid] <= n) lo = mid; else hi = mid - 1;
    }
    b = lo;
    const int T = row_tiles(seq_e[b]);
    const int loc = n - seq_base[b];
    g = div_by(loc, T, 1.0 / T);
    t = loc - g * T;
  };
  // the item after (b, g, t): next tile, next head, or next sequence with rows
  auto next_item = [&](int& b, int& g, int& t) {
    if (++t == row_tiles(seq_e[b])) {
      t = 0;
      if (++g == H) {
        g = 0;
        do ++b; while (b < a.bs && seq_e[b] == 0);
      }
    }
  };
  // tile of the first key any row of tile t of sequence b sees (sliding window)
  auto first_tile = [&](int b, int t) {
    return a.window > 0 ? max(0, seq_p[b] + div_by(t * BM, G, inv_g) - a.window) >> lbn : 0;
  };
  const int ipt = ceil_div(n_items, kThreads);  // items per thread, contiguous
  const int n0 = min(n_items, tid * ipt), n1 = min(n_items, n0 + ipt);

  // 2. cost of every item in KV tiles (keys up to the last token of its rows)
  //    and its running sum; cb holds the costs until the chunks are cut
  int my_total = 0;
  if (n0 < n1) {
    int b, g, t;
    decode(n0, b, g, t);
    for (int n = n0; n < n1; ++n) {
      const int row_hi = min((t + 1) * BM, seq_e[b] * G) - 1;
      // with a custom mask every key of the sequence may be seen
      const int keys =
          !a.masked ? seq_p[b] + div_by(row_hi, G, inv_g) + 1 : (a.prefix_lens ? seq_span[b] : seq_p[b] + seq_e[b]);
      // (at least one tile: size classes and chunk ranges assume it)
      const int cost = max(1, ((keys + BN - 1) >> lbn) - first_tile(b, t));
      cb[n] = cost;
      my_total += cost;
      next_item(b, g, t);
    }
  }
  int64_t total;
  {
    int v[1] = {my_total}, ex[1];
    int64_t tot[1];
    block_excl_scan<1>(v, ex, tot, sh, scan_no++ & 1);
    int run = ex[0];
    for (int n = n0; n < n1; ++n) {
      cum[n] = run;
      run += cb[n];
    }
    if (tid == 0) cum[n_items] = (int)tot[0];
    total = tot[0];
  }

  // 3. chunk limit: a 1/rounds share of the average work per resident
  //    workgroup (so that heaviest-first placement can even out the CUs),
  //    grown until the split chunks fit the partial-state budget; and
  // 4. with the limit that fits, in the same block scan: partial-slot and
  //    merge-record offsets of split items and the first chunk of every item
  // (the total fits 31 bits: cum holds its running sums)
  const int64_t shares = (int64_t)a.slots * (a.rounds > 0 ? a.rounds : 1);
  int chunk = (int)((total + shares - 1) / shares);
  if (chunk < a.min_chunk) chunk = a.min_chunk;
  double inv_chunk = 1.0 / chunk;
  auto pieces = [&](int c) { return c > chunk ? div_by(c - 1, chunk, inv_chunk) + 1 : 1; };
  int mcarry, n_chunks;
  for (;;) {
    int v[3] = {0, 0, 0}, ex[3];
    int64_t tot[3];
    for (int n = n0; n < n1; ++n) {
      const int k = pieces(cb[n]);
      v[0] += k > 1 ? k : 0;
      v[1] += k > 1 ? 1 : 0;
      v[2] += k;
    }
    block_excl_scan<3>(v, ex, tot, sh, scan_no++ & 1);
    if (tot[0] > a.part_budget) {
      chunk *= 2;
      inv_chunk = 1.0 / chunk;
      continue;
    }
    for (int n = n0; n < n1; ++n) {
      const int k = pieces(cb[n]);
      // partial bases < part_budget <= 4096 and merge indices < part_budget fit 16 bits each
      pm[n] = (ex[0] << 16) | ex[1];
      cb[n] = ex[2];  // from here on the item's cost is cum[n + 1] - cum[n]
      ex[0] += k > 1 ? k : 0;
      ex[1] += k > 1 ? 1 : 0;
      ex[2] += k;
    }
    if (tid == 0) cb[n_items] = (int)tot[2];
    mcarry = (int)tot[1];
    n_chunks = (int)tot[2];
    break;
  }
  __syncthreads();  // cum, pm and cb complete before the walks over chunks

  // 5. XCD bin of every chunk (midpoint rule), then heaviest first inside a bin
  // size class of a chunk of sz tiles (sizes are <= chunk); only orders
  // chunks, so the float rounding near class edges is harmless
  const float cls_scale = (float)kBuckets / (float)chunk;
  auto size_class = [&](int sz) { return min(kBuckets - 1, (int)((float)(sz - 1) * cls_scale)); };
  int X = a.xcds < 1 ? 1 : (a.xcds > kMaxXcd ? kMaxXcd : a.xcds);
  // With three or more chunks per resident workgroup, one heaviest-first
  // list dealt round-robin over the XCDs evens out the CUs better than
  // per-XCD ranges, and that outweighs the L2 sharing the ranges buy; with
  // fewer, the ranges' sharing of a sequence's K/V rows in one L2 wins.
  if ((int64_t)n_chunks >= 3 * (int64_t)a.slots) X = 1;
  // XCD of a chunk: which of X equal-cost ranges holds its midpoint (twice the
  // midpoint against twice the range ends; integer compares only)
  // (twice the total fits 32 bits unsigned)
  uint32_t bnd2[kMaxXcd];
  {
    // (x+1) total / X as (x+1)(q X + r) / X = (x+1) q + (x+1) r / X
    const double inv_x = 1.0 / X;
    const int q = div_by((int)total, X, inv_x);
    const int rem = (int)total - q * X;
#pragma unroll
    for (int x = 0; x < kMaxXcd; ++x) bnd2[x] = 2u * (uint32_t)((x + 1) * q + div_by((x + 1) * rem, X, inv_x));
  }
  auto bin_of = [&](int n, int k0, int k1) {
    const uint32_t mid2 = 2u * (uint32_t)cum[n] + (uint32_t)(k0 + k1);
    int x = 0;
#pragma unroll
    for (int i = 0; i < kMaxXcd - 1; ++i) x += (i < X - 1 && mid2 >= bnd2[i]) ? 1 : 0;
    return x;
  };
  // chunks in contiguous runs per thread; the item of the run's first chunk
  // is the last n with cb[n] <= j0.  Every item has at least one chunk, so
  // n <= cb[n] <= n + (n_chunks - n_items): that item lies in
  // [j0 - (n_chunks - n_items), j0] (one step when nothing is split)
  const int cpt = ceil_div(n_chunks, kThreads);
  const int j0 = min(n_chunks, tid * cpt), j1 = min(n_chunks, j0 + cpt);
  int n_first = 0;
  if (j0 < j1) {
    int lo = max(0, j0 - (n_chunks - n_items)), hi = min(n_items - 1, j0);
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cb[mid] <= j0) lo = mid; else hi = mid - 1;
    }
    n_first = lo;
  }
  // visit(n, b, g, t, s, k, k0, k1) for the thread's chunks in order: piece s
  // of the k of item n = (b, g, t), KV tiles k0 .. k1 - 1 of the item's range;
  // full chunks of `chunk` tiles and the remainder last (chunks of mixed sizes
  // let the heaviest-first placement fill the last round, where equal pieces
  // would quantise it)
  auto walk = [&](auto&& visit) {
    if (j0 >= j1) return;
    int n = n_first, b, g, t;
    decode(n, b, g, t);
    for (int j = j0; j < j1; ++j) {
      const int base = cb[n], k = cb[n + 1] - base, s = j - base;
      const int c = cum[n + 1] - cum[n];
      const int k0 = s * chunk;  // (0 when the item is whole)
      const int k1 = s + 1 == k ? c : (s + 1) * chunk;
      visit(n, b, g, t, s, k, k0, k1);
      if (s + 1 == k && ++n < n_items) next_item(b, g, t);
    }
  };
  constexpr int kPer = kMaxXcd * kBuckets / kThreads;  // counters per thread in the scan
  int max_count = 0, n_placed = 0;
  // chunks of bin x (bin_start as set by the last scan)
  auto bin_count = [&](int x) { return (x + 1 < X ? sh.bin_start[x + 1] : n_placed) - sh.bin_start[x]; };
  for (int attempt = 0; attempt < 2; ++attempt) {
    // (the first attempt's counters were zeroed at the start)
    walk([&](int n, int, int, int, int, int, int k0, int k1) {
      atomicAdd(&sh.bucket[bin_of(n, k0, k1) * kBuckets + (kBuckets - 1 - size_class(k1 - k0))], 1);
    });
    __syncthreads();
    // one exclusive scan over all (bin, class) counters, kPer per thread; a
    // bin's ranks are offsets from its first counter's scan value
    {
      int cnt[kPer], sum = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int idx = tid * kPer + i;
        cnt[i] = idx < X * kBuckets ? sh.bucket[idx] : 0;
        sum += cnt[i];
      }
      int v[1] = {sum}, ex[1];
      int64_t tot[1];
      block_excl_scan<1>(v, ex, tot, sh, scan_no++ & 1);
      int run = ex[0];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int idx = tid * kPer + i;
        if (idx < X * kBuckets) {
          sh.bucket[idx] = run;
          if (idx % kBuckets == 0) sh.bin_start[idx / kBuckets] = run;
        }
        run += cnt[i];
      }
      n_placed = (int)tot[0];
      __syncthreads();
    }
    max_count = 0;
    for (int x = 0; x < X; ++x) max_count = max(max_count, bin_count(x));
    if ((int64_t)max_count * X <= a.max_work || X == 1) break;
    X = 1;  // bins too uneven for the grid: plain heaviest-first order
    for (int i = tid; i < kMaxXcd * kBuckets; i += kThreads) sh.bucket[i] = 0;
    __syncthreads();
  }
  if (tid == 0) {
    a.hdr->num_work = max_count * X;  // grid slots in use, empty items included
    a.hdr->num_chunks = n_chunks;
    a.hdr->xcds = X;
    a.hdr->num_merge = mcarry;
    a.hdr->chunk_tiles = chunk;
    a.hdr->total_tiles = (int32_t)total;
    a.hdr->num_items = n_items;
  }
  walk([&](int n, int b, int g, int t, int s, int k, int k0, int k1) {
    const int x = bin_of(n, k0, k1);
    const int rank =
        atomicAdd(&sh.bucket[x * kBuckets + (kBuckets - 1 - size_class(k1 - k0))], 1) - sh.bin_start[x];
    const int pbase = (int)((uint32_t)pm[n] >> 16), midx = pm[n] & 0xFFFF;
    const int first = first_tile(b, t);
    WorkItem w;
    w.b = b;
    w.g = g;
    w.t = t;
    w.kt_begin = first + k0;
    w.kt_end = first + k1;
    w.part = k > 1 ? pbase + s : -1;
    w.merge = k > 1 ? midx : -1;
    w.pad0 = 0;
    // the sequence's keys: kv_indices serves j < n_idx; in a two-part call
    // the new tokens' rows follow (n_keys = P + E); in a unified call the
    // index span holds every key, of which a causal row sees at most P + E
    const int E = seq_e[b], P = seq_p[b], span = seq_span[b];
    w.q0 = seq_q0[b];
    w.E = E;
    w.kvs = seq_kvs[b];
    w.P = P;
    w.n_idx = a.prefix_lens ? (!a.masked ? min(span, P + E) : span) : span;
    w.n_keys = a.prefix_lens ? w.n_idx : span + E;
    w.pad1 = w.pad2 = 0;
    a.work[rank * X + x] = w;
    if (k > 1 && s == 0) {
      MergeItem m;
      m.b = b;
      m.g = g;
      m.t = t;
      m.part_base = pbase;
      m.n = k;
      m.q0 = w.q0;
      m.E = E;
      m.pad0 = 0;
      a.merge[midx] = m;
    }
  });
  // unused slots of shorter bins hold empty items (slot i = rank X + x):
  // b = -1 is all a workgroup reads of one before it returns
  for (int i = tid; i < max_count * X; i += kThreads) {
    if (i / X < bin_count(i % X)) continue;
    a.work[i].b = -1;
  }
}

__global__ __launch_bounds__(kThreads) void plan_kernel(PlanArgs a) {
  __shared__ Shared sh;
  // zero row read for keys past a sequence
  for (int i = threadIdx.x; i < kZeroRowBytes / 16; i += kThreads)
    reinterpret_cast<uint4*>(a.zero_row)[i] = make_uint4(0, 0, 0, 0);
  if (a.bs <= kSeqLds && a.max_items <= kItemLds)
    plan_body<true>(a, sh);
  else
    plan_body<false>(a, sh);
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  // the planner divides by the tile sizes with shifts
  if (a.bm <= 0 || a.bn <= 0 || (a.bm & (a.bm - 1)) != 0 || (a.bn & (a.bn - 1)) != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
