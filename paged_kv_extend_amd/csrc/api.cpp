// C ABI of libpkv.so: host-side argument checks, workspace sizing and the
// stream-ordered launch sequence of an extend call (plan, attention, then a
// merge launch that combines the chunks of split items).  Checks use only
// host-visible sizes, so no call reads device memory or waits for the device
// -- except in the debug build (PKV_DEBUG), which first checks the index
// arrays on the device and waits for the result.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <stddef.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kMinChunkTiles = 8;           // never split an item below this many KV tiles
constexpr size_t kPartialBytes = 64u << 20;  // budget for split partial states
// Items are cut into chunks of at most 1/kSplitRounds of the average work per
// resident workgroup.  Finer cuts even out the CUs on paper (llama8b's
// heaviest-first makespan is 13 % above the mean unsplit), but every extra
// chunk reloads its Q rows and writes and merges 128 KB of fp32 state: on
// one MI355X, 2 and 4 rounds made llama8b 10 % and 50 % slower.
constexpr int kSplitRounds = 1;
constexpr int kXcds = 8;                     // MI355X: 8 XCDs, workgroups dealt round-robin

// V is the first lv columns of K (same base pointers and strides), as in the
// MLA layout: the direct-load kernel then reads V out of the K tile.
// (without new-token tensors, as in a unified call, only the pool decides)
bool v_inside_k(const pkv_attn_desc_t& d, const void* k_extend, const void* v_extend, const void* k_pool,
                const void* v_pool) {
  const bool ext = (!k_extend && !v_extend) ||
                   (k_extend == v_extend && d.ke_stride_tok == d.ve_stride_tok && d.ke_stride_head == d.ve_stride_head);
  return d.lv <= d.lq && ext && k_pool == v_pool && d.kp_stride_slot == d.vp_stride_slot &&
         d.kp_stride_head == d.vp_stride_head;
}

// The attention kernel that serves (dtype, lq, lv), with V inside K or not,
// and its row / key tiling.  Automatic order: direct loads, register-staged.
enum class Kernel { kNone, kDl, kAttn };

std::atomic<int> g_prefer{0};  // Kernel preferred by extend_attention_prefer_kernel, 0 = automatic
// Split granularity set by extend_attention_set_split (0: the defaults above)
std::atomic<int> g_split_rounds{0};
std::atomic<int> g_min_chunk{0};

// Tiling of kernel k for the shape, or false when k does not serve it.
bool kernel_tiling(Kernel k, int dtype, int lq, int lv, bool v_in_k, pkv::Tiling* t) {
  switch (k) {
    case Kernel::kDl: return pkv::dl_tiling(dtype, lq, lv, v_in_k, t);
    case Kernel::kAttn: return pkv::attn_tiling(dtype, lq, lv, t);
    default: return false;
  }
}

Kernel pick_kernel(int dtype, int lq, int lv, bool v_in_k, pkv::Tiling* t) {
  const Kernel pref = static_cast<Kernel>(g_prefer.load(std::memory_order_relaxed));
  const auto serves = [&](Kernel k) { return kernel_tiling(k, dtype, lq, lv, v_in_k, t); };
  if (pref != Kernel::kNone && serves(pref)) return pref;
  for (Kernel k : {Kernel::kDl, Kernel::kAttn})
    if (serves(k)) return k;
  return Kernel::kNone;
}

const char* kernel_symbol(Kernel k) {
  switch (k) {
    case Kernel::kDl: return "attn_dl_kernel";
    case Kernel::kAttn: return "attn_kernel";
    default: return nullptr;
  }
}

// Resident attention workgroups on the current device, cached per (device, variant).
int resident_slots(int dtype, int lq, int lv, bool v_in_k) {
  static std::mutex mu;
  static std::unordered_map<long long, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  pkv::Tiling t;
  const Kernel k = pick_kernel(dtype, lq, lv, v_in_k, &t);
  const long long key = ((long long)dev << 36) | ((long long)k << 33) | ((long long)v_in_k << 32) |
                        ((long long)dtype << 24) | ((long long)lq << 12) | lv;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  int per_cu = 1;
  switch (k) {
    case Kernel::kDl: per_cu = pkv::dl_blocks_per_cu(lq, lv, v_in_k); break;
    default: per_cu = pkv::attention_blocks_per_cu(dtype, lq, lv); break;
  }
  const int slots = cus * per_cu;
  cache[key] = slots;
  return slots;
}

// Row and key tiling of the kernel serving (dtype, lq, lv) with or without V inside K.
bool tiling_for(const pkv_attn_desc_t& d, bool v_in_k, pkv::Tiling* t) {
  return pick_kernel(d.dtype, d.lq, d.lv, v_in_k, t) != Kernel::kNone;
}

// Sizes derived from the descriptor; returns 0 and sets the error when invalid.
int check_desc(const pkv_attn_desc_t* d, pkv::Tiling* t) {
  if (!d) return fail(PKV_ERR_INVALID, "desc is NULL");
  if (d->dtype != PKV_BF16 && d->dtype != PKV_FP32)
    return fail(PKV_ERR_UNSUPPORTED, "dtype %d is not PKV_BF16 or PKV_FP32", d->dtype);
  if (d->bs < 0) return fail(PKV_ERR_INVALID, "bs %d < 0", d->bs);
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID, "head counts must be positive (%d, %d)", d->num_q_heads, d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d", d->num_q_heads,
                d->num_kv_heads);
  // every head-dim pair that a V-inside-K variant serves has a general
  // variant too, so the general tiling decides what is supported
  if (!tiling_for(*d, false, t))
    return fail(PKV_ERR_UNSUPPORTED, "head dims (lq %d, lv %d) not supported for dtype %d", d->lq, d->lv,
                d->dtype);
  if (d->total_q_tokens < 0 || d->num_prefix_indices < 0 || d->pool_slots < 0)
    return fail(PKV_ERR_INVALID, "negative size (total_q_tokens %lld, num_prefix_indices %lld, pool_slots %lld)",
                (long long)d->total_q_tokens, (long long)d->num_prefix_indices, (long long)d->pool_slots);
  const int group = d->num_q_heads / d->num_kv_heads;
  if (d->total_q_tokens * (int64_t)group >= (1ll << 31) || d->num_prefix_indices >= (1ll << 31))
    return fail(PKV_ERR_UNSUPPORTED, "batch too large for 32-bit row indexing");
  if (d->num_prefix_indices > 0 && d->pool_slots <= 0)
    return fail(PKV_ERR_INVALID, "prefix indices given but pool_slots is %lld", (long long)d->pool_slots);
  const int64_t vec = d->dtype == PKV_BF16 ? 8 : 4;
  const int64_t strides[] = {d->q_stride_tok,   d->q_stride_head,  d->o_stride_tok,    d->o_stride_head,
                             d->ke_stride_tok,  d->ke_stride_head, d->ve_stride_tok,   d->ve_stride_head,
                             d->kp_stride_slot, d->kp_stride_head, d->vp_stride_slot,  d->vp_stride_head};
  for (int64_t s : strides)
    if (s < 0 || s % vec != 0)
      return fail(PKV_ERR_UNSUPPORTED, "strides must be non-negative multiples of %lld elements", (long long)vec);
  return PKV_OK;
}

pkv::PlanBounds plan_bounds(const pkv_attn_desc_t* d, const pkv::Tiling& t, size_t partial_bytes = kPartialBytes) {
  pkv::PlanBounds pb;
  const int64_t group = d->num_q_heads / d->num_kv_heads;
  // sum_b ceil(E_b G / BM) <= T G / BM + bs
  pb.max_items = (int64_t)d->num_kv_heads * (d->total_q_tokens * group / t.bm + d->bs + 1);
  int64_t budget = (int64_t)(partial_bytes / ((size_t)t.bm * (d->lv + 2) * sizeof(float)));
  if (budget > 4096) budget = 4096;
  if (budget < 16) budget = 16;
  pb.part_budget = budget;
  pb.max_merge = budget / 2;
  // chunks never exceed items + budget; placement may leave up to as many
  // empty slots again when the XCD bins end up uneven in count
  pb.max_work = 2 * (pb.max_items + budget) + 8;
  return pb;
}

pkv::WsLayout ws_layout(const pkv_attn_desc_t* d, const pkv::Tiling& t, const pkv::PlanBounds& pb) {
  pkv::WsLayout l;
  size_t off = 0;
  l.header = off;
  off = align_up(off + sizeof(pkv::PlanHeader), 256);
  l.zero_row = off;
  off = align_up(off + pkv::kZeroRowBytes, 256);
  l.work = off;
  off = align_up(off + sizeof(pkv::WorkItem) * (size_t)pb.max_work, 256);
  l.merge = off;
  off = align_up(off + sizeof(pkv::MergeItem) * (size_t)(pb.max_merge > 0 ? pb.max_merge : 1), 256);
  l.scratch = off;
  off = align_up(off + sizeof(int32_t) * (size_t)(6 * d->bs + 3 + 3 * pb.max_items), 256);
  l.part_ml = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)pb.part_budget * t.bm, 256);
  l.part_acc = off;
  off = align_up(off + sizeof(float) * (size_t)pb.part_budget * t.bm * d->lv, 256);
  l.total = off;
  return l;
}

#ifdef PKV_DEBUG
// Debug build: validate the index arrays on the device before anything reads
// them, then wait for the result (the one host sync of the library, in this
// build only).  flag: a device word of the workspace the launch sequence
// does not use yet.
int debug_check(int32_t* flag, const int32_t* qo_indptr, const int32_t* kv_indptr, const int64_t* kv_indices,
                const int32_t* prefix_lens, int32_t bs, int64_t total_q_tokens, int64_t num_indices,
                int64_t pool_slots, hipStream_t s) {
  if (bs <= 0) return PKV_OK;
  pkv::CheckArgs c;
  c.qo_indptr = qo_indptr;
  c.kv_indptr = kv_indptr;
  c.kv_indices = kv_indices;
  c.prefix_lens = prefix_lens;
  c.bs = bs;
  c.total_q_tokens = total_q_tokens;
  c.num_indices = num_indices;
  c.pool_slots = pool_slots;
  c.flag = flag;
  hipError_t e = hipMemsetAsync(flag, 0, sizeof(int32_t), s);
  if (e == hipSuccess) e = pkv::launch_check_indices(c, s);
  int32_t bad = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&bad, flag, sizeof bad, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "debug index check: %s", hipGetErrorString(e));
  if (bad)
    return fail(PKV_ERR_RANGE, "debug index check failed:%s%s%s%s", (bad & 1) ? " qo_indptr" : "",
                (bad & 2) ? " kv_indptr" : "", (bad & 4) ? " a slot outside [0, pool_slots)" : "",
                (bad & 8) ? " a negative prefix_lens" : "");
  return PKV_OK;
}
#endif

// Event pairs around attention launches while profiling is enabled.
struct Profile {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs;
  size_t used = 0;
};
Profile& profile() {
  static Profile p;
  return p;
}
constexpr size_t kMaxProfiled = 4096;

// Returns the event pair to record around this call's attention kernel, or nulls.
std::pair<hipEvent_t, hipEvent_t> profile_slot() {
  Profile& p = profile();
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.on || p.used >= kMaxProfiled) return {nullptr, nullptr};
  if (p.used == p.pairs.size()) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess) return {nullptr, nullptr};
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return {nullptr, nullptr};
    }
    p.pairs.push_back({a, b});
  }
  return p.pairs[p.used++];
}

}  // namespace

extern "C" {

int pkv_profile_enable(int on) {
  Profile& p = profile();
  std::lock_guard<std::mutex> lk(p.mu);
  p.on = on != 0;
  if (p.on) p.used = 0;
  return ok();
}

int pkv_profile_read(double* total_ms, int64_t* calls) {
  if (!total_ms || !calls) return fail(PKV_ERR_INVALID, "NULL output");
  Profile& p = profile();
  std::lock_guard<std::mutex> lk(p.mu);
  double t = 0.0;
  for (size_t i = 0; i < p.used; ++i) {
    if (hipEventSynchronize(p.pairs[i].second) != hipSuccess)
      return fail(PKV_ERR_HIP, "event synchronize failed");
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, p.pairs[i].first, p.pairs[i].second) != hipSuccess)
      return fail(PKV_ERR_HIP, "event elapsed time failed");
    t += ms;
  }
  *total_ms = t;
  *calls = (int64_t)p.used;
  return ok();
}

const char* pkv_last_error(void) { return g_err; }

#ifdef PKV_DEBUG
const char* pkv_version(void) { return "pkv 0.2.0 (gfx950, debug: index checks)"; }
#else
const char* pkv_version(void) { return "pkv 0.2.0 (gfx950)"; }
#endif

const char* extend_attention_kernel_name(const pkv_attn_desc_t* desc, const void* k_extend, const void* v_extend,
                                         const void* k_pool, const void* v_pool) {
  pkv::Tiling t;
  if (check_desc(desc, &t) != PKV_OK) return nullptr;
  const bool vk = v_inside_k(*desc, k_extend, v_extend, k_pool, v_pool);
  return kernel_symbol(pick_kernel(desc->dtype, desc->lq, desc->lv, vk, &t));
}

int build_unified_kv_indices(const int32_t* prefix_kv_indptr, const int64_t* prefix_kv_indices,
                             const int32_t* extend_start_loc, const int32_t* extend_seq_lens,
                             const int64_t* extend_kv_indices, int32_t bs, int64_t num_prefix_indices,
                             int64_t num_extend_indices, int32_t* unified_kv_indptr,
                             int64_t* unified_kv_indices, int64_t capacity, int32_t* prefix_lens,
                             void* stream) {
  if (bs < 0) return fail(PKV_ERR_INVALID, "bs %d < 0", bs);
  if (num_prefix_indices < 0 || num_extend_indices < 0 || capacity < 0)
    return fail(PKV_ERR_INVALID, "negative length");
  if (!unified_kv_indptr) return fail(PKV_ERR_INVALID, "unified_kv_indptr is NULL");
  if (bs > 0 && (!prefix_kv_indptr || !extend_start_loc || !extend_seq_lens))
    return fail(PKV_ERR_INVALID, "an input indptr/length array is NULL");
  if ((num_prefix_indices > 0 && !prefix_kv_indices) || (num_extend_indices > 0 && !extend_kv_indices))
    return fail(PKV_ERR_INVALID, "an input index array is NULL");
  if (num_prefix_indices + num_extend_indices >= (1ll << 31))
    return fail(PKV_ERR_UNSUPPORTED, "more than 2^31 - 1 indices");
  if (capacity < num_prefix_indices + num_extend_indices)
    return fail(PKV_ERR_CAPACITY, "capacity %lld < %lld prefix + %lld extend indices", (long long)capacity,
                (long long)num_prefix_indices, (long long)num_extend_indices);
  if (capacity > 0 && !unified_kv_indices) return fail(PKV_ERR_INVALID, "unified_kv_indices is NULL");
  hipError_t e = pkv::launch_index_build(prefix_kv_indptr, prefix_kv_indices, extend_start_loc, extend_seq_lens,
                                         extend_kv_indices, bs, unified_kv_indptr, unified_kv_indices,
                                         prefix_lens, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "index build launch: %s", hipGetErrorString(e));
  return ok();
}

int store_kv_cache(const void* k_extend, const void* v_extend, void* k_pool, void* v_pool,
                   const int64_t* out_cache_loc, const pkv_attn_desc_t* desc, void* stream) {
  pkv::Tiling t;
  int rc = check_desc(desc, &t);
  if (rc != PKV_OK) return rc;
  const pkv_attn_desc_t& d = *desc;
  if (d.total_q_tokens == 0) return ok();
  if (!k_extend || !v_extend || !k_pool || !v_pool || !out_cache_loc)
    return fail(PKV_ERR_INVALID, "k_extend / v_extend / k_pool / v_pool / out_cache_loc is NULL");
  if (d.pool_slots <= 0) return fail(PKV_ERR_INVALID, "pool_slots is %lld", (long long)d.pool_slots);
  const void* ptrs[] = {k_extend, v_extend, k_pool, v_pool};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(PKV_ERR_UNSUPPORTED, "tensor base pointers must be 16-byte aligned");
  const int64_t e = d.dtype == PKV_BF16 ? 2 : 4;
  const bool vk = v_inside_k(d, k_extend, v_extend, k_pool, v_pool);
  pkv::StoreArgs a;
  a.k_ext = static_cast<const char*>(k_extend);
  a.v_ext = static_cast<const char*>(v_extend);
  a.k_pool = static_cast<char*>(k_pool);
  a.v_pool = static_cast<char*>(v_pool);
  a.loc = out_cache_loc;
  a.ke_st = d.ke_stride_tok * e;
  a.ke_sh = d.ke_stride_head * e;
  a.ve_st = d.ve_stride_tok * e;
  a.ve_sh = d.ve_stride_head * e;
  a.kp_ss = d.kp_stride_slot * e;
  a.kp_sh = d.kp_stride_head * e;
  a.vp_ss = d.vp_stride_slot * e;
  a.vp_sh = d.vp_stride_head * e;
  a.ck = (uint32_t)(d.lq * e / 16);
  a.cv = vk ? 0u : (uint32_t)(d.lv * e / 16);  // V inside K: its bytes travel with the K row
  const int64_t rows = d.total_q_tokens * d.num_kv_heads;
  if (rows * (int64_t)(a.ck + a.cv) >= (1ll << 31)) return fail(PKV_ERR_UNSUPPORTED, "too many rows to store");
  a.rows = (uint32_t)rows;
  a.hkv = (uint32_t)d.num_kv_heads;
  hipError_t he = pkv::launch_store_kv(a, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(PKV_ERR_HIP, "store launch: %s", hipGetErrorString(he));
  return ok();
}

int gather_kv_indices(const int32_t* req_to_token, int64_t req_to_token_stride, const int64_t* req_pool_indices,
                      const int32_t* kv_lens, const int32_t* kv_start_idx, int32_t bs, int32_t* kv_indptr,
                      int64_t* kv_indices, int64_t capacity, void* stream) {
  if (bs < 0 || req_to_token_stride < 0 || capacity < 0) return fail(PKV_ERR_INVALID, "negative size");
  if (!kv_indptr) return fail(PKV_ERR_INVALID, "kv_indptr is NULL");
  if (bs > 0 && (!req_to_token || !req_pool_indices || !kv_lens))
    return fail(PKV_ERR_INVALID, "req_to_token / req_pool_indices / kv_lens is NULL");
  if (capacity > 0 && !kv_indices) return fail(PKV_ERR_INVALID, "kv_indices is NULL");
  if (capacity >= (1ll << 31)) return fail(PKV_ERR_UNSUPPORTED, "more than 2^31 - 1 indices");
  pkv::GatherArgs a;
  a.req_to_token = req_to_token;
  a.stride = req_to_token_stride;
  a.req_pool_indices = req_pool_indices;
  a.kv_lens = kv_lens;
  a.kv_start_idx = kv_start_idx;
  a.bs = bs;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.capacity = capacity;
  hipError_t he = pkv::launch_gather_indices(a, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(PKV_ERR_HIP, "gather launch: %s", hipGetErrorString(he));
  return ok();
}

int extend_attention_prefer_kernel(const char* name) {
  if (!name) return fail(PKV_ERR_INVALID, "kernel name is NULL");
  static const struct {
    const char* name;
    Kernel k;
  } names[] = {{"auto", Kernel::kNone}, {"dl", Kernel::kDl}, {"attn", Kernel::kAttn}};
  for (const auto& n : names)
    if (strcmp(name, n.name) == 0) {
      g_prefer.store(static_cast<int>(n.k), std::memory_order_relaxed);
      return ok();
    }
  return fail(PKV_ERR_INVALID, "unknown kernel \"%s\" (auto, dl, attn)", name);
}

int extend_attention_set_split(int rounds, int min_chunk_tiles) {
  if (rounds < 0 || rounds > 64 || min_chunk_tiles < 0 || min_chunk_tiles > (1 << 20))
    return fail(PKV_ERR_INVALID, "split rounds %d (0..64) or minimum chunk %d tiles (0..2^20) out of range", rounds,
                min_chunk_tiles);
  g_split_rounds.store(rounds, std::memory_order_relaxed);
  g_min_chunk.store(min_chunk_tiles, std::memory_order_relaxed);
  return ok();
}

size_t extend_attention_workspace_size(const pkv_attn_desc_t* desc) {
  pkv::Tiling t;
  if (check_desc(desc, &t) != PKV_OK) return 0;
  g_err[0] = '\0';
  // the kernel, and with it the row tiling, depends on whether V lies inside
  // K (which only the call shows) and on the kernel preference: size for
  // every kernel that could serve the shape
  size_t total = 0;
  for (Kernel k : {Kernel::kDl, Kernel::kAttn})
    for (bool vk : {false, true}) {
      pkv::Tiling tk;
      if (kernel_tiling(k, desc->dtype, desc->lq, desc->lv, vk, &tk))
        total = std::max(total, ws_layout(desc, tk, plan_bounds(desc, tk)).total);
    }
  return total;
}

}  // extern "C"

namespace {

// The workspace of extend_attention_fwd_noalloc: one array per device, held
// until the process ends.  Its name is a host-side stand-in; the device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = 32u << 20;
constexpr size_t kNoAllocPartialBytes = 24u << 20;  // of it, for split chunks' partial states
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array into *out; returns
// PKV_OK or an error code (message set).
int device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, "device %d beyond the %d the no-allocation entry point serves", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress of the scratch array: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

// Both entry points: two-part when prefix_lens is NULL (new tokens' K/V from
// k_extend / v_extend), unified otherwise (every key through kv_indices).
// partial_bytes bounds the split chunks' partial states; noalloc: the
// workspace is the current device's scratch array, of workspace_bytes
// (no profiling events).
int attention_call(const void* q_extend, const void* k_extend, const void* v_extend, void* o, const void* k_pool,
                   const void* v_pool, const int32_t* qo_indptr, const int32_t* kv_indptr,
                   const int64_t* kv_indices, const int32_t* prefix_lens, float sm_scale, float logit_cap,
                   const pkv_attn_desc_t* desc, void* workspace, size_t workspace_bytes, void* stream,
                   size_t partial_bytes = kPartialBytes, bool noalloc = false) {
  pkv::Tiling t;
  int rc = check_desc(desc, &t);
  if (rc != PKV_OK) return rc;
  const pkv_attn_desc_t& d = *desc;
  const bool unified = prefix_lens != nullptr;
  if (!std::isfinite(sm_scale) || std::isnan(logit_cap))
    return fail(PKV_ERR_INVALID, "sm_scale must be finite and logit_cap not NaN");
  if (d.bs == 0 || d.total_q_tokens == 0) return ok();  // no query rows: nothing to write
  if (!qo_indptr || !kv_indptr) return fail(PKV_ERR_INVALID, "qo_indptr / kv_indptr is NULL");
  if (!q_extend || !o) return fail(PKV_ERR_INVALID, "q_extend / o is NULL");
  if (!unified && (!k_extend || !v_extend)) return fail(PKV_ERR_INVALID, "k_extend / v_extend is NULL");
  if (unified) k_extend = v_extend = nullptr;  // not read
  if (d.num_prefix_indices > 0 && (!kv_indices || !k_pool || !v_pool))
    return fail(PKV_ERR_INVALID, "kv_indices / k_pool / v_pool is NULL with a non-empty index array");
  if (d.custom_mask && !d.mask_indptr) return fail(PKV_ERR_INVALID, "custom_mask without mask_indptr");
  const void* ptrs[] = {q_extend, k_extend, v_extend, o, k_pool, v_pool};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(PKV_ERR_UNSUPPORTED, "tensor base pointers must be 16-byte aligned");

  const bool vk = v_inside_k(d, k_extend, v_extend, k_pool, v_pool);
  if (vk) tiling_for(d, true, &t);  // the tiling of the kernel that serves this call
  const pkv::PlanBounds pb = plan_bounds(&d, t, partial_bytes);
  const pkv::WsLayout wl = ws_layout(&d, t, pb);
  if (noalloc) {
    if (wl.total > workspace_bytes)
      return fail(PKV_ERR_UNSUPPORTED,
                  "batch too large for the no-allocation entry point: %zu bytes of planning and partial state "
                  "needed, its scratch array holds %zu",
                  wl.total, workspace_bytes);
    rc = device_scratch(&workspace);
    if (rc != PKV_OK) return rc;
  }
  if (!workspace || workspace_bytes < wl.total)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                wl.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  char* ws = static_cast<char*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int group = d.num_q_heads / d.num_kv_heads;
#ifdef PKV_DEBUG
  rc = debug_check(reinterpret_cast<int32_t*>(ws + wl.header + offsetof(pkv::PlanHeader, pad)), qo_indptr,
                   kv_indptr, kv_indices, prefix_lens, d.bs, d.total_q_tokens, d.num_prefix_indices, d.pool_slots, s);
  if (rc != PKV_OK) return rc;
#endif

  pkv::PlanArgs pa;
  pa.qo_indptr = qo_indptr;
  pa.kv_indptr = kv_indptr;
  pa.prefix_lens = prefix_lens;
  pa.window = d.sliding_window > 0 ? d.sliding_window : 0;
  pa.masked = d.custom_mask != nullptr;
  pa.bs = d.bs;
  pa.num_kv_heads = d.num_kv_heads;
  pa.group = group;
  pa.bm = t.bm;
  pa.bn = t.bn;
  pa.slots = resident_slots(d.dtype, d.lq, d.lv, vk);
  const int forced_rounds = g_split_rounds.load(std::memory_order_relaxed);
  const int forced_min = g_min_chunk.load(std::memory_order_relaxed);
  pa.min_chunk = forced_min > 0 ? forced_min : kMinChunkTiles;
  pa.rounds = forced_rounds > 0 ? forced_rounds : kSplitRounds;
  pa.xcds = kXcds;
  pa.max_work = pb.max_work;
  pa.max_items = pb.max_items;
  pa.part_budget = pb.part_budget;
  pa.max_merge = pb.max_merge;
  pa.hdr = reinterpret_cast<pkv::PlanHeader*>(ws + wl.header);
  pa.zero_row = ws + wl.zero_row;
  pa.work = reinterpret_cast<pkv::WorkItem*>(ws + wl.work);
  pa.merge = reinterpret_cast<pkv::MergeItem*>(ws + wl.merge);
  pa.scratch = reinterpret_cast<int32_t*>(ws + wl.scratch);
  hipError_t e = pkv::launch_plan(pa, s);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "plan launch: %s", hipGetErrorString(e));

  const double scale = sm_scale != 0.0f ? (double)sm_scale : 1.0 / sqrt((double)d.lq);
  const double log2e = 1.4426950408889634;
  pkv::AttnArgs a;
  a.q = q_extend;
  a.k_ext = k_extend;
  a.v_ext = v_extend;
  a.o = o;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.qo_indptr = qo_indptr;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.prefix_lens = prefix_lens;
  a.window = pa.window;
  a.sinks = d.sinks;
  a.custom_mask = d.custom_mask;
  a.mask_indptr = d.mask_indptr;
  a.q_st = d.q_stride_tok;
  a.q_sh = d.q_stride_head;
  a.o_st = d.o_stride_tok;
  a.o_sh = d.o_stride_head;
  a.ke_st = d.ke_stride_tok;
  a.ke_sh = d.ke_stride_head;
  a.ve_st = d.ve_stride_tok;
  a.ve_sh = d.ve_stride_head;
  a.kp_ss = d.kp_stride_slot;
  a.kp_sh = d.kp_stride_head;
  a.vp_ss = d.vp_stride_slot;
  a.vp_sh = d.vp_stride_head;
  a.group = group;
  a.use_cap = logit_cap > 0.0f ? 1 : 0;
  a.neg_q = scale < 0.0 ? 1 : 0;
  a.scale_log2 = (float)(fabs(scale) * log2e);
  a.cap_in = logit_cap > 0.0f ? (float)(fabs(scale) / logit_cap) : 0.0f;
  a.cap_out = logit_cap > 0.0f ? (float)(logit_cap * log2e) : 0.0f;
  a.zero_row = pa.zero_row;
  a.hdr = pa.hdr;
  a.work = pa.work;
  a.merge = pa.merge;
  a.part_acc = reinterpret_cast<float*>(ws + wl.part_acc);
  a.part_ml = reinterpret_cast<float*>(ws + wl.part_ml);
  const auto ev = noalloc ? std::pair<hipEvent_t, hipEvent_t>{nullptr, nullptr} : profile_slot();
  if (ev.first) (void)hipEventRecord(ev.first, s);
  pkv::Tiling td;
  switch (pick_kernel(d.dtype, d.lq, d.lv, vk, &td)) {
    case Kernel::kDl: e = pkv::launch_dl(d.lq, d.lv, vk, a, pb.max_work, s); break;
    default: e = pkv::launch_attention(d.dtype, d.lq, d.lv, a, pb.max_work, s); break;
  }
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  if (ev.second) (void)hipEventRecord(ev.second, s);
  // the chunks of split items, merged after the launch that wrote them
  e = pkv::launch_split_merge(d.dtype, d.lv, pa.bm, a, s);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int extend_attention_fwd(const void* q_extend, const void* k_extend, const void* v_extend, void* o,
                         const void* k_pool, const void* v_pool, const int32_t* qo_indptr,
                         const int32_t* kv_indptr, const int64_t* kv_indices, float sm_scale,
                         float logit_cap, const pkv_attn_desc_t* desc, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return attention_call(q_extend, k_extend, v_extend, o, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices,
                        nullptr, sm_scale, logit_cap, desc, workspace, workspace_bytes, stream);
}

int extend_attention_fwd_unified(const void* q_extend, void* o, const void* k_pool, const void* v_pool,
                                 const int32_t* qo_indptr, const int32_t* unified_kv_indptr,
                                 const int64_t* unified_kv_indices, const int32_t* prefix_lens,
                                 float sm_scale, float logit_cap, const pkv_attn_desc_t* desc,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!prefix_lens && desc && desc->bs > 0 && desc->total_q_tokens > 0)
    return fail(PKV_ERR_INVALID, "prefix_lens is NULL");
  static const int32_t kNoPrefix = 0;  // never read: the call returns before any launch
  return attention_call(q_extend, nullptr, nullptr, o, k_pool, v_pool, qo_indptr, unified_kv_indptr,
                        unified_kv_indices, prefix_lens ? prefix_lens : &kNoPrefix, sm_scale, logit_cap, desc,
                        workspace, workspace_bytes, stream);
}

size_t extend_attention_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int extend_attention_fwd_noalloc(const void* q_extend, const void* k_extend, const void* v_extend, void* o,
                                 const void* k_pool, const void* v_pool, const int32_t* qo_indptr,
                                 const int32_t* kv_indptr, const int64_t* kv_indices, float sm_scale,
                                 float logit_cap, const pkv_attn_desc_t* desc, void* stream) {
  pkv::Tiling t;
  int rc = check_desc(desc, &t);
  if (rc != PKV_OK) return rc;
  if (desc->bs == 0 || desc->total_q_tokens == 0) return ok();  // no query rows: nothing to write
  // the scratch array is taken inside, once the sizes are known to fit; nothing
  // in it needs to start at zero: the planner writes the plan header, the
  // zero row and every work item, and each partial state is written before
  // the merge reads it
  return attention_call(q_extend, k_extend, v_extend, o, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices,
                        nullptr, sm_scale, logit_cap, desc, nullptr, kNoAllocScratchBytes, stream,
                        kNoAllocPartialBytes, true);
}

}  // extern "C"

// ---------------------------------------------------------------- decode
namespace {

// Workgroups the decode launch aims at: MI355X has 256 CUs and a decode
// workgroup fills one (its LDS ring), so one round of equal chunks streams
// longest with the fewest pipeline fills and partial states (measured best
// against 512 .. 2048).  A function of the sizes only, so that the workspace
// size query and the call agree on any device.
constexpr int64_t kDecodeTargetWgs = 256;
constexpr int64_t kDecodeMinChunk = 128;
constexpr int64_t kDecodeMaxChunk = 16384;
constexpr int64_t kMaxGridY = 65535;

struct DecodeSizes {
  int hblocks, gh_count;
  int64_t chunk, chunks;
  size_t vis, part_ml, part_acc, total;  // workspace offsets and size
};

DecodeSizes decode_sizes(const pkv_attn_desc_t& d) {
  DecodeSizes z;
  const int group = d.num_q_heads / d.num_kv_heads;
  z.hblocks = (group + 15) / 16;
  z.gh_count = d.num_kv_heads * z.hblocks;
  int64_t vis = d.num_prefix_indices;  // visible keys over all requests, at most
  if (d.sliding_window > 0) vis = std::min(vis, (int64_t)d.bs * ((int64_t)d.sliding_window + 1));
  int64_t chunk = (vis * z.gh_count + kDecodeTargetWgs - 1) / kDecodeTargetWgs;
  chunk = std::max(chunk, (vis + kMaxGridY - 1) / kMaxGridY);
  chunk = std::min(std::max(chunk, kDecodeMinChunk), std::max(kDecodeMaxChunk, (vis + kMaxGridY - 1) / kMaxGridY));
  chunk = (chunk + 63) / 64 * 64;
  z.chunk = chunk;
  z.chunks = (vis + chunk - 1) / chunk;
  const int64_t rows = 2 * z.chunks * z.gh_count * 16;  // two partial pieces per chunk
  size_t off = 0;
  z.vis = off;
  off = align_up(off + sizeof(int32_t) * (size_t)(d.bs + 1), 256);
  z.part_ml = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)rows, 256);
  z.part_acc = off;
  off = align_up(off + sizeof(float) * (size_t)rows * d.lv, 256);
  z.total = off;
  return z;
}

// Whether a decode kernel variant serves the batch (bf16, listed head dims).
bool decode_kernel_serves(const pkv_attn_desc_t& d) {
  int waves = 0;
  return pkv::decode_supported(d.dtype, d.lq, d.lv, false, &waves) ||
         pkv::decode_supported(d.dtype, d.lq, d.lv, true, &waves);
}

// A decode batch that no decode kernel serves (fp32, other head dims) runs as
// the unified extend of one new token per request whose prefix is every
// earlier key, all of them read through kv_indices.
pkv_attn_desc_t decode_as_extend(const pkv_attn_desc_t& d) {
  pkv_attn_desc_t e = d;
  e.total_q_tokens = d.bs;
  e.ke_stride_tok = e.ke_stride_head = e.ve_stride_tok = e.ve_stride_head = 0;
  return e;
}

// Bytes before the extend workspace on that route: qo_indptr[bs + 1] and
// prefix_lens[bs].
size_t decode_rows_bytes(const pkv_attn_desc_t& d) {
  return align_up(sizeof(int32_t) * (size_t)(2 * (int64_t)d.bs + 1), 256);
}

int check_decode_desc(const pkv_attn_desc_t* d) {
  if (!d) return fail(PKV_ERR_INVALID, "desc is NULL");
  if (d->bs < 0) return fail(PKV_ERR_INVALID, "bs %d < 0", d->bs);
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID, "head counts must be positive (%d, %d)", d->num_q_heads, d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d", d->num_q_heads,
                d->num_kv_heads);
  if (d->custom_mask) return fail(PKV_ERR_UNSUPPORTED, "decode attention takes no custom mask");
  if (d->num_prefix_indices < 0 || d->pool_slots < 0)
    return fail(PKV_ERR_INVALID, "negative size (num_prefix_indices %lld, pool_slots %lld)",
                (long long)d->num_prefix_indices, (long long)d->pool_slots);
  if (d->num_prefix_indices >= (1ll << 31)) return fail(PKV_ERR_UNSUPPORTED, "more than 2^31 - 1 keys");
  if (d->bs > 65535) return fail(PKV_ERR_UNSUPPORTED, "decode batch of %d requests exceeds 65535", d->bs);
  if (d->num_prefix_indices > 0 && d->pool_slots <= 0)
    return fail(PKV_ERR_INVALID, "keys given but pool_slots is %lld", (long long)d->pool_slots);
  if (!decode_kernel_serves(*d)) {
    // the extend kernels' own limits (dtype, head dims, strides) apply
    pkv::Tiling t;
    const pkv_attn_desc_t e = decode_as_extend(*d);
    return check_desc(&e, &t);
  }
  const int64_t strides[] = {d->q_stride_tok, d->q_stride_head, d->o_stride_tok, d->o_stride_head,
                             d->kp_stride_slot, d->kp_stride_head, d->vp_stride_slot, d->vp_stride_head};
  for (int64_t s : strides)
    if (s < 0 || s % 8 != 0) return fail(PKV_ERR_UNSUPPORTED, "strides must be non-negative multiples of 8 elements");
  return PKV_OK;
}

}  // namespace

extern "C" {

size_t decode_attention_workspace_size(const pkv_attn_desc_t* desc) {
  if (check_decode_desc(desc) != PKV_OK) return 0;
  g_err[0] = '\0';
  if (!decode_kernel_serves(*desc)) {
    const pkv_attn_desc_t e = decode_as_extend(*desc);
    return decode_rows_bytes(*desc) + extend_attention_workspace_size(&e);
  }
  return decode_sizes(*desc).total;
}

int decode_attention_fwd(const void* q, void* o, const void* k_pool, const void* v_pool, const int32_t* kv_indptr,
                         const int64_t* kv_indices, float sm_scale, float logit_cap, const pkv_attn_desc_t* desc,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_decode_desc(desc);
  if (rc != PKV_OK) return rc;
  const pkv_attn_desc_t& d = *desc;
  if (!std::isfinite(sm_scale) || std::isnan(logit_cap))
    return fail(PKV_ERR_INVALID, "sm_scale must be finite and logit_cap not NaN");
  if (d.bs == 0) return ok();
  if (!kv_indptr || !q || !o) return fail(PKV_ERR_INVALID, "kv_indptr / q / o is NULL");
  if (d.num_prefix_indices > 0 && (!kv_indices || !k_pool || !v_pool))
    return fail(PKV_ERR_INVALID, "kv_indices / k_pool / v_pool is NULL with a non-empty index array");
  const void* ptrs[] = {q, o, k_pool, v_pool};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(PKV_ERR_UNSUPPORTED, "tensor base pointers must be 16-byte aligned");
  if (!decode_kernel_serves(d)) {
    const pkv_attn_desc_t e = decode_as_extend(d);
    const size_t rows = decode_rows_bytes(d);
    const size_t need = rows + extend_attention_workspace_size(&e);
    g_err[0] = '\0';
    if (!workspace || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                  need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    int32_t* qo_indptr = static_cast<int32_t*>(workspace);
    int32_t* prefix_lens = qo_indptr + d.bs + 1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e1 = pkv::launch_decode_rows(kv_indptr, d.bs, qo_indptr, prefix_lens, s);
    if (e1 != hipSuccess) return fail(PKV_ERR_HIP, "decode rows launch: %s", hipGetErrorString(e1));
    rc = attention_call(q, nullptr, nullptr, o, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, prefix_lens,
                        sm_scale, logit_cap, &e, static_cast<char*>(workspace) + rows, workspace_bytes - rows,
                        stream);
    if (rc != PKV_OK) return rc;
    // a request without keys has no visible key: its output row is zero
    e1 = pkv::launch_decode_zero_empty(kv_indptr, d.bs, d.num_q_heads, d.lv, d.dtype == PKV_FP32 ? 4 : 2, o,
                                       d.o_stride_tok, d.o_stride_head, s);
    if (e1 != hipSuccess) return fail(PKV_ERR_HIP, "decode zero launch: %s", hipGetErrorString(e1));
    return ok();
  }
  // V inside K: the variant that reads V out of the K tile when there is one;
  // the general variant reads the same rows twice otherwise
  int waves = 0;
  bool vk = v_inside_k(d, nullptr, nullptr, k_pool, v_pool);
  if (vk && !pkv::decode_supported(d.dtype, d.lq, d.lv, true, &waves)) vk = false;
  if (!pkv::decode_supported(d.dtype, d.lq, d.lv, vk, &waves))
    return fail(PKV_ERR_UNSUPPORTED, "head dims (lq %d, lv %d) not supported for decode", d.lq, d.lv);
  const DecodeSizes z = decode_sizes(d);
  if (!workspace || workspace_bytes < z.total)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                z.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  char* ws = static_cast<char*>(workspace);
#ifdef PKV_DEBUG
  rc = debug_check(reinterpret_cast<int32_t*>(ws + z.part_ml), nullptr, kv_indptr, kv_indices, nullptr, d.bs, d.bs,
                   d.num_prefix_indices, d.pool_slots, reinterpret_cast<hipStream_t>(stream));
  if (rc != PKV_OK) return rc;
#endif
  const double scale = sm_scale != 0.0f ? (double)sm_scale : 1.0 / sqrt((double)d.lq);
  const double log2e = 1.4426950408889634;
  pkv::DecodeArgs a;
  a.q = q;
  a.o = o;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.sinks = d.sinks;
  a.q_st = d.q_stride_tok;
  a.q_sh = d.q_stride_head;
  a.o_st = d.o_stride_tok;
  a.o_sh = d.o_stride_head;
  a.kp_ss = d.kp_stride_slot * 2;
  a.kp_sh = d.kp_stride_head * 2;
  a.vp_ss = d.vp_stride_slot * 2;
  a.vp_sh = d.vp_stride_head * 2;
  a.bs = d.bs;
  a.group = d.num_q_heads / d.num_kv_heads;
  a.hblocks = z.hblocks;
  a.gh_count = z.gh_count;
  a.chunk = (int32_t)z.chunk;
  a.window = d.sliding_window > 0 ? d.sliding_window : 0;
  a.use_cap = logit_cap > 0.0f;
  a.scale_log2 = (float)(scale * log2e);
  a.cap_in = a.use_cap ? (float)(scale / logit_cap) : 0.0f;
  a.cap_out = a.use_cap ? (float)(logit_cap * log2e) : 0.0f;
  a.vis = reinterpret_cast<int32_t*>(ws + z.vis);
  a.part_ml = reinterpret_cast<float*>(ws + z.part_ml);
  a.part_acc = reinterpret_cast<float*>(ws + z.part_acc);
  const auto ev = profile_slot();
  hipError_t e = pkv::launch_decode(d.lq, d.lv, vk, a, z.chunks, reinterpret_cast<hipStream_t>(stream), ev.first,
                                    ev.second);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
