// Internal declarations shared by the library's translation units.
// Nothing here is part of the public ABI (include/pkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// One unit of attention work: packed query rows [t*BM, (t+1)*BM) of sequence
// b and KV head g, over KV tiles [kt_begin, kt_end) of the concatenated
// (prefix, new tokens) key sequence.  Packed row r is new token r / G, query
// head g*G + r % G (token-major, so one KV tile serves all G heads of a token).
// part < 0: the item covers all KV tiles and writes o directly; otherwise it is
// one chunk of a split item and writes unnormalised partial state into
// partial slot `part`.  b < 0 marks an empty slot.
// (an empty placement slot has b = -1 and nothing else written)
struct WorkItem {
  int32_t b, g, t, kt_begin, kt_end, part;
  int32_t merge;  // merge record of a split item's chunk, else -1
  int32_t pad0;
  // sequence b's keys as the planner read them from the index pointers, so
  // that a workgroup's first loads depend on this record alone
  int32_t q0, E;      // first new-token row, new tokens
  int32_t kvs, P;     // first index of the sequence, prefix keys
  int32_t n_idx;      // keys read through kv_indices: j < n_idx
  int32_t n_keys;     // keys that exist: j < n_keys
  int32_t pad1, pad2;
};

// A split item whose chunks occupy partial slots [part_base, part_base + n).
struct MergeItem {
  int32_t b, g, t, part_base, n;
  int32_t q0, E;  // sequence b's first new-token row and new tokens
  int32_t pad0;
};

// Planner output header at the start of the workspace.
struct PlanHeader {
  int32_t num_work;
  int32_t num_merge;
  int32_t chunk_tiles;  // split threshold the planner settled on
  int32_t total_tiles;  // KV tiles over all items before splitting
  int32_t num_items;    // items before splitting
  int32_t num_chunks;   // work items after splitting (num_work also counts empty slots)
  int32_t xcds;         // XCD bins used for placement (1: plain heaviest-first)
  int32_t pad[57];
};

constexpr int kZeroRowBytes = 4096;  // >= 576 fp32 or bf16 elements

// Static tiling of one kernel instantiation.
struct Tiling {
  int bm;       // packed query rows per workgroup
  int bn;       // keys per KV tile
  int threads;  // workgroup size
};

// Upper bounds that size the workspace (functions of host-visible sizes only).
struct PlanBounds {
  int64_t max_items;    // items before splitting
  int64_t max_work;     // items after splitting
  int64_t part_budget;  // partial slots available for split chunks
  int64_t max_merge;    // split items
};

// Workspace carve-up.
struct WsLayout {
  size_t header, zero_row, work, merge, scratch, part_ml, part_acc, total;
};

struct AttnArgs {
  const void* q;
  const void* k_ext;
  const void* v_ext;
  void* o;
  const void* k_pool;
  const void* v_pool;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int64_t* kv_indices;
  // NULL: two-part call (kv_indices hold the prefix, new tokens' K/V are
  // k_ext / v_ext rows).  Else unified call: kv_indices hold every key and
  // prefix_lens[b] of sequence b's keys are prefix keys.
  const int32_t* prefix_lens;
  int32_t window;       // > 0: sliding window (keys j < P + i - window hidden)
  const float* sinks;   // [num_q_heads] sink logits (natural units), or NULL
  const uint8_t* custom_mask;  // byte per (query, key) replacing the causal rule, or NULL
  const int64_t* mask_indptr;  // [bs] first byte of sequence b's [E, n_keys] matrix
  int64_t q_st, q_sh, o_st, o_sh, ke_st, ke_sh, ve_st, ve_sh, kp_ss, kp_sh, vp_ss, vp_sh;
  int32_t group;     // query heads per KV head
  int32_t use_cap;   // soft-cap enabled
  int32_t neg_q;     // the scale is negative: q is negated (exact) and |scale| used
  float scale_log2;  // |scale| * log2(e): logits are kept in base-2 units
  float cap_in;      // |scale| / cap
  float cap_out;     // cap * log2(e)
  const void* zero_row;  // >= max(lq, lv) zero elements, read for keys past a sequence
  const PlanHeader* hdr;
  const WorkItem* work;
  MergeItem* merge;
  float* part_acc;   // [part][bm][lv]
  float* part_ml;    // [part][bm][2]: running max (base-2 units), sum of weights
};

struct PlanArgs {
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* prefix_lens;  // as in AttnArgs
  int32_t window;              // as in AttnArgs
  int32_t masked;              // a custom mask: every key of a sequence may be seen
  int32_t bs, num_kv_heads, group, bm, bn;
  int32_t slots;          // workgroups resident at once on the device
  int32_t min_chunk;      // never split below this many KV tiles
  int32_t rounds;         // chunk limit = average work per resident workgroup / rounds
  int32_t xcds;           // XCDs to spread work over (workgroup i runs on XCD i mod xcds)
  int64_t max_items, part_budget, max_merge;
  int64_t max_work;       // grid size: slots available for work items
  PlanHeader* hdr;
  void* zero_row;    // zeroed by the planner: kZeroRowBytes bytes
  WorkItem* work;    // [max_work]
  MergeItem* merge;  // [max_merge]
  int32_t* scratch;  // [6 * bs + 3 + 3 * max_items], used when the batch exceeds the LDS arrays
};

// Keys of sequence b as the attention kernels see them.
//  Two-part call: P = prefix indices of b (keys j < P through kv_indices),
//    keys P .. P+E-1 are new-token rows; n_idx = P, n_keys = P + E.
//  Unified call (page extend_attention.py, _fwd_kernel_unified): every key j
//    < span goes through kv_indices, P = prefix_lens[b]; keys at or past P + E
//    are never visible, so n_idx = n_keys = min(span, P + E), which also keeps
//    every index read inside the sequence's own span.
// A query at new-token position i sees key j iff j < n_keys and j <= P + i
// (causal), or, with a custom mask (causal == false), iff j < n_keys and its
// mask byte is set; a unified call then keeps the whole span.
// "no sliding window": a first visible key below every key
constexpr int kNoLowerKey = -(1 << 30);

struct SeqKeys {
  int q0, E;   // first new-token row, new tokens
  int kvs, P;  // first index of the sequence, prefix keys
  int n_idx;   // keys read through kv_indices: j < n_idx
  int n_keys;  // keys that exist: j < n_keys
};
__device__ __forceinline__ SeqKeys item_keys(const WorkItem& it) {
  SeqKeys k;
  k.q0 = it.q0;
  k.E = it.E;
  k.kvs = it.kvs;
  k.P = it.P;
  k.n_idx = it.n_idx;
  k.n_keys = it.n_keys;
  return k;
}

// Kernel variants: (dtype, lq, lv).  Returns false when unsupported.
bool attn_tiling(int dtype, int lq, int lv, Tiling* t);
hipError_t launch_attention(int dtype, int lq, int lv, const AttnArgs& a, int64_t grid,
                            hipStream_t s);
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
// Merge of the chunks of split items (after the attention launch; bm = rows per item).
hipError_t launch_split_merge(int dtype, int lv, int bm, const AttnArgs& a, hipStream_t s);
// KV-cache store: byte strides; ck / cv = 16-byte chunks of a K / V row
// (cv = 0 when V lies inside K and is stored with it); rows = tokens * hkv.
struct StoreArgs {
  const char* k_ext;
  const char* v_ext;
  char* k_pool;
  char* v_pool;
  const int64_t* loc;  // [tokens] pool slot of each new token
  int64_t ke_st, ke_sh, ve_st, ve_sh, kp_ss, kp_sh, vp_ss, vp_sh;
  uint32_t rows, hkv, ck, cv;
};
hipError_t launch_store_kv(const StoreArgs& a, hipStream_t s);

// Request-to-token index gather.
struct GatherArgs {
  const int32_t* req_to_token;      // [rows, stride]
  int64_t stride;
  const int64_t* req_pool_indices;  // [bs]
  const int32_t* kv_lens;           // [bs]
  const int32_t* kv_start_idx;      // [bs] or NULL
  int32_t bs;
  int32_t* kv_indptr;               // [bs + 1] out
  int64_t* kv_indices;              // [capacity] out
  int64_t capacity;
};
hipError_t launch_gather_indices(const GatherArgs& a, hipStream_t s);

// Index validation (launched by the debug build only).  The kv_indices read
// are [kv_indptr[0], kv_indptr[bs]); flag gets bits set for each kind of
// violation (qo_indptr 1, kv_indptr 2, slot 4, prefix_lens 8).
struct CheckArgs {
  const int32_t* qo_indptr;    // [bs + 1] or NULL (decode)
  const int32_t* kv_indptr;    // [bs + 1]
  const int64_t* kv_indices;
  const int32_t* prefix_lens;  // [bs] or NULL
  int32_t bs;
  int64_t total_q_tokens;      // bound of qo_indptr[bs]
  int64_t num_indices;         // bound of kv_indptr[bs] - kv_indptr[0]
  int64_t pool_slots;
  int32_t* flag;               // device word, zero before the launch
};
hipError_t launch_check_indices(const CheckArgs& a, hipStream_t s);

hipError_t launch_index_build(const int32_t* prefix_kv_indptr, const int64_t* prefix_kv_indices,
                              const int32_t* extend_start_loc, const int32_t* extend_seq_lens,
                              const int64_t* extend_kv_indices, int32_t bs,
                              int32_t* unified_kv_indptr, int64_t* unified_kv_indices,
                              int32_t* prefix_lens, hipStream_t s);
// Decode attention (one query token per request over its pool keys).
struct DecodeArgs {
  const void* q;     // [bs, num_q_heads, lq], strides (q_st, q_sh) elements
  void* o;           // [bs, num_q_heads, lv], strides (o_st, o_sh) elements
  const void* k_pool;
  const void* v_pool;
  const int32_t* kv_indptr;   // [bs + 1]
  const int64_t* kv_indices;  // pool slot of each key
  const float* sinks;         // [num_q_heads] sink logits (natural units), or NULL
  int64_t q_st, q_sh, o_st, o_sh;
  int64_t kp_ss, kp_sh, vp_ss, vp_sh;  // BYTES
  int32_t bs, group, hblocks;
  int32_t gh_count;  // num_kv_heads * hblocks: the x extent of the grid
  int32_t chunk;     // keys per chunk (a multiple of 64)
  int32_t window;    // > 0: only the last window + 1 keys of a request are seen
  int32_t use_cap;
  float scale_log2;  // scale * log2(e)
  float cap_in;      // scale / cap
  float cap_out;     // cap * log2(e)
  int32_t* vis;      // [bs + 1] first visible key of request b among all requests' visible keys
  float* part_ml;    // [2 * chunks][gh_count][16][2]: max (base-2 units), sum of weights
  float* part_acc;   // [2 * chunks][gh_count][16][lv]
};
// (dtype, lq, lv, V inside K) served by the decode kernel; waves per workgroup.
bool decode_supported(int dtype, int lq, int lv, bool v_in_k, int* waves);
// fp32 decode through the unified extend: row arrays (qo_indptr[b] = b,
// prefix_lens[b] = keys - 1) and, afterwards, zero outputs of keyless requests.
hipError_t launch_decode_rows(const int32_t* kv_indptr, int32_t bs, int32_t* qo_indptr, int32_t* prefix_lens,
                              hipStream_t s);
hipError_t launch_decode_zero_empty(const int32_t* kv_indptr, int32_t bs, int32_t hq, int32_t lv, int32_t elem_bytes,
                                    void* o, int64_t o_st, int64_t o_sh, hipStream_t s);
// Plan launch, then the attention launch over `chunks` chunks of a.chunk keys
// and the merge launch; non-null events are recorded on s around the last two.
hipError_t launch_decode(int lq, int lv, bool v_in_k, const DecodeArgs& a, int64_t chunks, hipStream_t s,
                         hipEvent_t before, hipEvent_t after);

// Workgroups of the attention kernel resident per CU (from the occupancy API).
int attention_blocks_per_cu(int dtype, int lq, int lv);
// The direct-to-LDS kernel (bf16, head dims 64, 128, 256, and 576/512 when V is
// the first lv columns of K); preferred when it applies.
bool dl_tiling(int dtype, int lq, int lv, bool v_in_k, Tiling* t);
hipError_t launch_dl(int lq, int lv, bool v_in_k, const AttnArgs& a, int64_t grid, hipStream_t s);
int dl_blocks_per_cu(int lq, int lv, bool v_in_k);

}  // namespace pkv
