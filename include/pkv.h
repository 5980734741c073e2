/*
 * pkv.h -- C ABI of the paged-KV extend-attention library (libpkv.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * Extend attention is prefill with a cached prefix: every new ("extend")
 * token of a sequence attends to the sequence's cached prefix, read from a
 * token-granular KV pool through slot indices, and causally to the new
 * tokens of its own sequence.  The operations follow the SGLang pages on
 * the subject: page "extend_attention.py" (sglang 0.5.3rc2 -> 0.5.4.post1
 * diff) and page "flashinfer_backend.py" (blame view).
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers, owned by the caller; the
 *    library allocates nothing and keeps no state between calls (it caches
 *    device properties only).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and is asynchronous.  No call waits for the device or copies device data
 *    to the host, so every call may be captured into a HIP graph.
 *  - Arguments are checked on the host only, from the sizes passed in.  A
 *    non-zero return means nothing was enqueued; pkv_last_error() then holds a
 *    message.  Values inside device arrays (lengths, slots) are trusted: they
 *    must be consistent with the sizes passed in, as documented per argument.
 *  - Index/offset arrays: indptr and length arrays are int32, slot index
 *    arrays are int64.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define PKV_OK 0
#define PKV_ERR_INVALID (-1)     /* null pointer, negative size, inconsistent sizes */
#define PKV_ERR_UNSUPPORTED (-2) /* dtype, head dims, stride or alignment not supported */
#define PKV_ERR_WORKSPACE (-3)   /* workspace missing or smaller than the size query */
#define PKV_ERR_CAPACITY (-4)    /* output index buffer too small */
#define PKV_ERR_HIP (-5)         /* a HIP runtime call or kernel launch failed */
#define PKV_ERR_RANGE (-6)       /* index or indptr out of range: debug build (libpkv_debug.so) only */

/* Element types of q / k / v / o and the pools. */
#define PKV_BF16 0
#define PKV_FP32 1

/*
 * Unified KV index build.
 * Page "extend_attention.py": build_unified_kv_indices and
 * _copy_unified_indices_kernel.  For b in [0, bs):
 *   prefix_lens[b]          = prefix_kv_indptr[b+1] - prefix_kv_indptr[b]
 *   unified_kv_indptr[0]    = 0
 *   unified_kv_indptr[b+1]  = unified_kv_indptr[b] + prefix_lens[b] + extend_seq_lens[b]
 *   unified_kv_indices[unified_kv_indptr[b] + o] =
 *       prefix_kv_indices[prefix_kv_indptr[b] + o]               for o <  prefix_lens[b]
 *       extend_kv_indices[extend_start_loc[b] + o - prefix_lens[b]] otherwise
 *
 * Arguments (device pointers unless noted):
 *  prefix_kv_indptr   int32[bs+1], non-decreasing; need not start at 0.
 *  prefix_kv_indices  int64[num_prefix_indices]; read at
 *                     [prefix_kv_indptr[0], prefix_kv_indptr[bs]).
 *  extend_start_loc   int32[>= bs]; only the first bs entries are read.
 *  extend_seq_lens    int32[>= bs], >= 0; only the first bs entries are read.
 *  extend_kv_indices  int64[num_extend_indices].
 *  bs                 host int, >= 0; bs == 0 writes unified_kv_indptr[0] = 0 only.
 *  num_prefix_indices, num_extend_indices
 *                     host ints: lengths of the two input index arrays.
 *  unified_kv_indptr  out int32[bs+1].
 *  unified_kv_indices out int64[capacity]; entries at and past
 *                     unified_kv_indptr[bs] are not written.
 *  capacity           host int; must be >= num_prefix_indices + num_extend_indices
 *                     (the page sizes its output the same way, so no device
 *                     value has to be read on the host), else PKV_ERR_CAPACITY.
 *  prefix_lens        out int32[bs], or NULL when not wanted.
 *  stream             hipStream_t.
 * The caller guarantees that every sequence's slices lie inside the input
 * arrays and that the total fits int32.
 */
int build_unified_kv_indices(const int32_t* prefix_kv_indptr, const int64_t* prefix_kv_indices,
                             const int32_t* extend_start_loc, const int32_t* extend_seq_lens,
                             const int64_t* extend_kv_indices, int32_t bs,
                             int64_t num_prefix_indices, int64_t num_extend_indices,
                             int32_t* unified_kv_indptr, int64_t* unified_kv_indices,
                             int64_t capacity, int32_t* prefix_lens, void* stream);

/*
 * Prefix index gather from the request-to-token table.
 * Page "flashinfer_backend.py": create_flashinfer_kv_indices_triton, and the
 * running sum kv_indptr[1:bs+1] = cumsum(paged_kernel_lens) of
 * call_begin_forward (computed here on the device).  For b in [0, bs):
 *   kv_indptr[0] = 0, kv_indptr[b+1] = kv_indptr[b] + kv_lens[b]
 *   kv_indices[kv_indptr[b] + o] = req_to_token[req_pool_indices[b] * req_to_token_stride + s_b + o]
 *   for o < kv_lens[b], s_b = kv_start_idx[b] (0 when kv_start_idx is NULL).
 * The table holds int32 slots (as the page's request-to-token pool does); the
 * indices are written as int64, the type extend_attention_fwd reads.
 *
 * Arguments (device pointers unless noted):
 *  req_to_token       int32[rows * req_to_token_stride] (row-major table).
 *  req_to_token_stride host int, >= 0: elements between table rows.
 *  req_pool_indices   int64[bs], table rows.
 *  kv_lens            int32[bs], >= 0.
 *  kv_start_idx       int32[bs] or NULL.
 *  bs                 host int, >= 0; bs == 0 writes kv_indptr[0] = 0 only.
 *  kv_indptr          out int32[bs+1].
 *  kv_indices         out int64[capacity]; nothing at or past capacity is
 *                     written, whatever the lengths hold.
 *  capacity           host int >= 0: the sum of kv_lens, as the caller
 *                     sizes the output (the page's paged_kernel_lens_sum).
 * The caller guarantees that every request's run lies inside the table.
 */
int gather_kv_indices(const int32_t* req_to_token, int64_t req_to_token_stride, const int64_t* req_pool_indices,
                      const int32_t* kv_lens, const int32_t* kv_start_idx, int32_t bs, int32_t* kv_indptr,
                      int64_t* kv_indices, int64_t capacity, void* stream);

/*
 * Shapes and strides of one extend-attention call.  Strides are in
 * ELEMENTS; the last dimension of every tensor is contiguous.
 *
 *  q_extend  [total_q_tokens, num_q_heads, lq]   strides (q_stride_tok, q_stride_head)
 *  k_extend  [total_q_tokens, num_kv_heads, lq]  strides (ke_stride_tok, ke_stride_head)
 *  v_extend  [total_q_tokens, num_kv_heads, lv]  strides (ve_stride_tok, ve_stride_head)
 *  o         [total_q_tokens, num_q_heads, lv]   strides (o_stride_tok, o_stride_head)
 *  k_pool    [pool_slots, num_kv_heads, lq]      strides (kp_stride_slot, kp_stride_head)
 *  v_pool    [pool_slots, num_kv_heads, lv]      strides (vp_stride_slot, vp_stride_head)
 *
 * v_pool / v_extend may be views into k_pool / k_extend (the MLA layout on
 * page "cpu_graph_runner.py", qkv_proj_with_rope: V is the first lv columns
 * of the joint latent+rope K row).  Supported (lq, lv): (64,64), (80,80),
 * (96,96), (112,112), (128,128), (160,160), (192,192), (256,256), (192,128),
 * (288,256), (576,512) for bf16; (64,64), (128,128) for fp32.  Plain head
 * dims between the served tile widths run in the next wider tile with the
 * extra columns zero (page "extend_attention.py",
 * _get_block_sizes_for_extend_attention: the head dim is padded to a power
 * of two and the columns past Lq masked).  Strides must be multiples of 8
 * elements (bf16) or 4 (fp32) and base pointers 16-byte aligned.
 */
typedef struct {
  int32_t dtype; /* PKV_BF16 or PKV_FP32: q, k/v extend, pools and o share it */
  int32_t bs;
  int32_t num_q_heads;
  int32_t num_kv_heads; /* must divide num_q_heads */
  int32_t lq;           /* head dim of q and k */
  int32_t lv;           /* head dim of v and o */
  int64_t total_q_tokens;     /* qo_indptr[bs]; if the device arrays hold more new-token rows than this,
                                 the call plans no work and leaves o unwritten */
  int64_t num_prefix_indices; /* kv_indptr[bs] - kv_indptr[0] (length of kv_indices) */
  int64_t pool_slots;
  int64_t q_stride_tok, q_stride_head;
  int64_t o_stride_tok, o_stride_head;
  int64_t ke_stride_tok, ke_stride_head;
  int64_t ve_stride_tok, ve_stride_head;
  int64_t kp_stride_slot, kp_stride_head;
  int64_t vp_stride_slot, vp_stride_head;
  /* Options of page "extend_attention.py", _fwd_kernel_unified (zero-initialise
   * the struct to leave them off): */
  int32_t sliding_window; /* W > 0: new token i also sees no key j < P_b + i - W */
  int32_t pad0;
  const float* sinks;     /* DEVICE float32[num_q_heads] sink logits, or NULL:
                             exp(sinks[h] - max) joins the softmax denominator
                             of query head h (logits after scale and cap) */
  const uint8_t* custom_mask; /* DEVICE bytes, or NULL: replaces the causal rule.
                             Sequence b's keys j < L_b (L_b = P_b + E_b for
                             extend_attention_fwd, the index span for the
                             unified entry) are seen by new token i iff
                             custom_mask[mask_indptr[b] + i * L_b + j] != 0 */
  const int64_t* mask_indptr; /* DEVICE int64[bs], with custom_mask */
} pkv_attn_desc_t;

/*
 * Bytes of device workspace extend_attention_fwd needs for `desc` (a
 * function of the sizes only).  Returns 0 when desc is invalid; then
 * pkv_last_error() says why.
 */
size_t extend_attention_workspace_size(const pkv_attn_desc_t* desc);

/*
 * Extend attention forward.
 * Page "extend_attention.py": _fwd_kernel_unified (causal mask, scale,
 * soft-cap, online softmax, GQA head mapping) and extend_attention_fwd
 * (default scale); page "flashinfer_backend.py": forward_extend and
 * call_begin_forward (prefix read through kv_indptr / kv_indices, the new
 * tokens' K/V rows addressed by qo_indptr).
 *
 * For sequence b (P_b = kv_indptr[b+1] - kv_indptr[b] prefix tokens,
 * E_b = qo_indptr[b+1] - qo_indptr[b] new tokens), new token i in [0, E_b),
 * query head h and its KV head g = h / (num_q_heads / num_kv_heads):
 *   key j < P_b   : k_pool[kv_indices[kv_indptr[b] + j], g], v_pool likewise
 *   key j >= P_b  : k_extend[qo_indptr[b] + j - P_b, g], v_extend likewise
 *   visible keys  : j <= P_b + i
 *   s_j = scale * <q[qo_indptr[b] + i, h], K_j>, scale = sm_scale, or
 *         1/sqrt(lq) when sm_scale == 0;
 *   if logit_cap > 0: s_j = logit_cap * tanh(s_j / logit_cap)
 *   o[qo_indptr[b] + i, h] = sum_j softmax(s)_j V_j over the visible keys.
 * The K/V of the new tokens are NOT written into the pool here.
 *
 * Arguments (device pointers unless noted):
 *  q_extend, k_extend, v_extend, k_pool, v_pool: as in pkv_attn_desc_t.
 *  o           out, as in pkv_attn_desc_t; rows of every new token are written.
 *  qo_indptr   int32[bs+1], qo_indptr[0] == 0, non-decreasing, qo_indptr[bs]
 *              == desc->total_q_tokens.
 *  kv_indptr   int32[bs+1], non-decreasing, kv_indptr[bs] - kv_indptr[0] ==
 *              desc->num_prefix_indices.
 *  kv_indices  int64[num_prefix_indices], each in [0, pool_slots).
 *  sm_scale, logit_cap: host floats (see above).
 *  desc        host pointer.
 *  workspace   device buffer of >= extend_attention_workspace_size(desc)
 *              bytes, 256-byte aligned; contents need no initialisation and
 *              are scratch after the call.  Calls that overlap in time must
 *              use different workspaces.
 *  stream      hipStream_t.
 * The result does not depend on the order of sequences in the batch or on
 * which pool slots hold the prefix; it is bitwise reproducible run to run
 * on the same device.
 */
int extend_attention_fwd(const void* q_extend, const void* k_extend, const void* v_extend,
                         void* o, const void* k_pool, const void* v_pool,
                         const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int64_t* kv_indices, float sm_scale, float logit_cap,
                         const pkv_attn_desc_t* desc, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * KV-cache store of the new tokens.
 * Page "flashinfer_backend.py": forward_extend stores the new tokens' K/V
 * into the pool (set_kv_buffer(layer, cache_loc, k, v)) before the paged
 * attention reads it:
 *   k_pool[out_cache_loc[t], g, :lq] = k_extend[t, g, :lq]
 *   v_pool[out_cache_loc[t], g, :lv] = v_extend[t, g, :lv]
 * for t < desc->total_q_tokens and every KV head g; other slots are left
 * alone.  When V lies inside K (the MLA layout, see pkv_attn_desc_t) the K
 * row carries it and is written once.
 *
 * Arguments (device pointers unless noted):
 *  k_extend, v_extend, k_pool, v_pool: as in pkv_attn_desc_t (q and o strides
 *              of desc are not used).
 *  out_cache_loc int64[total_q_tokens], each in [0, pool_slots), distinct.
 *  desc        host pointer, checked as for extend_attention_fwd.
 *  stream      hipStream_t.
 */
int store_kv_cache(const void* k_extend, const void* v_extend, void* k_pool, void* v_pool,
                   const int64_t* out_cache_loc, const pkv_attn_desc_t* desc, void* stream);

/*
 * Unified one-stage extend attention.
 * Page "extend_attention.py": extend_attention_fwd_unified and
 * _fwd_kernel_unified.  Every key of a sequence, prefix and new tokens alike,
 * is read from the pool through one index array -- the arrays
 * build_unified_kv_indices produces -- so the new tokens' K/V must already be
 * stored in the pool at their slots.
 *
 * For sequence b (L_b = unified_kv_indptr[b+1] - unified_kv_indptr[b] keys,
 * P_b = prefix_lens[b], E_b = qo_indptr[b+1] - qo_indptr[b]), new token i in
 * [0, E_b), query head h and KV head g = h / (num_q_heads / num_kv_heads):
 *   key j in [0, L_b) : k_pool[unified_kv_indices[unified_kv_indptr[b] + j], g], v_pool likewise
 *   visible keys      : j < P_b (prefix) or j - P_b <= i (new tokens up to the query)
 *   scale, soft-cap and softmax as in extend_attention_fwd.
 * With L_b = P_b + E_b and the new tokens' rows stored at their slots this is
 * the two-part result of extend_attention_fwd.
 *
 * Arguments (device pointers unless noted):
 *  q_extend, o, k_pool, v_pool: as in pkv_attn_desc_t (the ke / ve strides of
 *              desc are not used).
 *  qo_indptr   int32[bs+1], as in extend_attention_fwd.
 *  unified_kv_indptr  int32[bs+1], non-decreasing; unified_kv_indptr[bs] -
 *              unified_kv_indptr[0] == desc->num_prefix_indices (the length
 *              of the index array).
 *  unified_kv_indices int64[num_prefix_indices], each in [0, pool_slots).
 *  prefix_lens int32[bs], 0 <= prefix_lens[b] <= L_b.  Keys at or past
 *              P_b + E_b are never visible and never read; a row that sees no
 *              key (L_b == 0) gets an undefined value.
 *  sm_scale, logit_cap, desc, workspace, workspace_bytes, stream: as in
 *              extend_attention_fwd (the same workspace size query applies).
 * Returns as extend_attention_fwd; prefix_lens == NULL with work to do is
 * PKV_ERR_INVALID.
 */
int extend_attention_fwd_unified(const void* q_extend, void* o, const void* k_pool, const void* v_pool,
                                 const int32_t* qo_indptr, const int32_t* unified_kv_indptr,
                                 const int64_t* unified_kv_indices, const int32_t* prefix_lens,
                                 float sm_scale, float logit_cap, const pkv_attn_desc_t* desc,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention: one new token per request over its pool keys.
 * Page "flashinfer_backend.py": forward_decode (each request's single query
 * token attends to every key its decode indices list, the new token's own
 * K/V already stored in the pool) and the decode index updater (kv_indptr /
 * kv_indices per request; with a sliding window only the last window + 1
 * keys).  Scale, soft-cap and sinks as in page "extend_attention.py",
 * _fwd_kernel_unified.  This equals extend_attention_fwd_unified with one new
 * token per request whose prefix is every earlier key; a kernel of its own
 * serves it, splitting each request's keys over many workgroups.
 *
 * For request b (n_b = kv_indptr[b+1] - kv_indptr[b] keys), query head h and
 * KV head g = h / (num_q_heads / num_kv_heads):
 *   key j in [f_b, n_b): k_pool[kv_indices[kv_indptr[b] + j], g], v_pool likewise,
 *       f_b = max(0, n_b - 1 - sliding_window) with a window, else 0
 *   s_j = scale * <q[b, h], K_j>, scale = sm_scale, or 1/sqrt(lq) when 0;
 *   if logit_cap > 0: s_j = logit_cap * tanh(s_j / logit_cap)
 *   o[b, h] = sum_j e^{s_j - m} V_j / (sum_j e^{s_j - m} + e^{sinks[h] - m})
 *   (the sink term only with desc->sinks); o[b, h] = 0 when n_b == 0.
 *
 * Arguments (device pointers unless noted):
 *  q          [bs, num_q_heads, lq]  strides (desc->q_stride_tok, q_stride_head)
 *  o          out [bs, num_q_heads, lv]  strides (o_stride_tok, o_stride_head);
 *             every row of every request is written.
 *  k_pool, v_pool: as in pkv_attn_desc_t; v_pool may be the first lv columns
 *             of k_pool (same base and strides; required for lq 576 / lv 512
 *             unless v_pool is a pool of its own).
 *  kv_indptr  int32[bs+1], non-decreasing, need not start at 0;
 *             desc->num_prefix_indices >= kv_indptr[bs] - kv_indptr[0] (the
 *             keys of the batch; a larger value only enlarges the launch and
 *             the workspace, a smaller one leaves keys unread).
 *  kv_indices int64, read at [kv_indptr[0], kv_indptr[bs]), each in
 *             [0, pool_slots).
 *  sm_scale, logit_cap: host floats as for extend_attention_fwd.
 *  desc       host pointer: bs <= 65535; sliding_window and sinks are
 *             honoured, custom_mask must be NULL; total_q_tokens and the
 *             k/v_extend strides are not used.  The decode kernels serve
 *             PKV_BF16 with (lq, lv) one of (64, 64), (128, 128), (256, 256),
 *             (192, 128), (288, 256), (576, 512); any other batch that
 *             extend_attention_fwd_unified serves (PKV_FP32, other head
 *             dims) runs as that call with one new token per request whose
 *             prefix is every earlier key, under the same rule as above and
 *             the extend limits on dtype, head dims and strides.
 *  workspace  device buffer of >= decode_attention_workspace_size(desc)
 *             bytes, 256-byte aligned, no initialisation needed; calls that
 *             overlap in time must use different workspaces.
 *  stream     hipStream_t.
 * The result is bitwise reproducible run to run on the same device.
 */
size_t decode_attention_workspace_size(const pkv_attn_desc_t* desc);
int decode_attention_fwd(const void* q, void* o, const void* k_pool, const void* v_pool, const int32_t* kv_indptr,
                         const int64_t* kv_indices, float sm_scale, float logit_cap, const pkv_attn_desc_t* desc,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * extend_attention_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation, kernels and
 * arguments as extend_attention_fwd, with the plan, the work list and the
 * split chunks' partial states kept in a scratch array of the library's own,
 * extend_attention_noalloc_scratch_bytes() = 32 MiB per device, which each
 * device the library runs on holds until the process ends.  The call itself
 * allocates nothing and calls no allocating routine.  Partial states get at
 * most 24 MiB of it (long key ranges are then split less finely than with a
 * full workspace: the result is the same up to rounding).
 *
 * Every call on one device shares that device's array: calls whose work
 * overlaps on one device (several streams, several host threads) race and
 * give undefined results; calls ordered on one stream are safe.  Nothing in
 * the array needs clearing between calls (each call writes what it reads).
 *
 * Returns as extend_attention_fwd, plus PKV_ERR_UNSUPPORTED when the batch's
 * planning state would not fit the array (at 32 query heads over 8 KV heads
 * and head dim 128, 16 sequences: more than about 470 000 new tokens) or for a device
 * index >= 64.
 */
int extend_attention_fwd_noalloc(const void* q_extend, const void* k_extend, const void* v_extend, void* o,
                                 const void* k_pool, const void* v_pool, const int32_t* qo_indptr,
                                 const int32_t* kv_indptr, const int64_t* kv_indices, float sm_scale,
                                 float logit_cap, const pkv_attn_desc_t* desc, void* stream);
size_t extend_attention_noalloc_scratch_bytes(void);

/*
 * Process-wide kernel preference for later extend_attention_fwd calls, for
 * tests and benchmarks: "auto" (the default: the fastest measured kernel that
 * serves the shape), "dl" (direct global-to-LDS loads; bf16, plain head dims
 * 64 to 256 and 576/512 with V inside K), "attn" (register-staged; fp32 64
 * and 128, bf16 64, 128, 256, 192/128, 288/256 and 576/512).  A
 * preferred kernel that does not serve a call's shape is passed over for the
 * automatic choice.  Results of every kernel meet the same accuracy bounds;
 * workspaces sized by extend_attention_workspace_size fit any choice.
 * Returns PKV_OK, or PKV_ERR_INVALID for an unknown name.  Not synchronised
 * with calls in flight on other host threads.
 */
int extend_attention_prefer_kernel(const char* name);

/*
 * Process-wide split granularity of later extend calls, for tests and
 * benchmarks.  The planner cuts a work item (sequence, KV head, row tile)
 * whose key range is longer than 1/rounds of the average work per resident
 * workgroup into chunks of keys, never shorter than min_chunk_tiles key
 * tiles; each chunk writes a partial softmax state (m, l, acc) and a merge
 * launch combines them in chunk order (page "flashinfer_backend.py",
 * forward_extend: the ragged and paged parts merged with merge_state).  The
 * result is the same softmax at any granularity, up to rounding.  0 keeps a
 * default (1 round, 8 tiles).  Chunks past the workspace's partial-state
 * budget are not made: the limit grows until the split fits.  Returns PKV_OK,
 * or PKV_ERR_INVALID for rounds outside 0..64 or min_chunk_tiles outside
 * 0..2^20.  Not synchronised with calls in flight on other host threads.
 */
int extend_attention_set_split(int rounds, int min_chunk_tiles);

/*
 * Name of the attention kernel symbol that serves a call with `desc` and these
 * K/V base pointers ("attn_dl_kernel" or "attn_kernel", as
 * profilers list it; pass NULL new-token pointers for a unified call),
 * or NULL when desc is invalid.  The pointers are only compared (V inside K
 * selects a variant), never dereferenced.  For matching profiler output;
 * results do not depend on it.
 */
const char* extend_attention_kernel_name(const pkv_attn_desc_t* desc, const void* k_extend, const void* v_extend,
                                         const void* k_pool, const void* v_pool);

/*
 * Measurement hook (not needed for results).  pkv_profile_enable(1) clears
 * the record and makes every later extend_attention_fwd,
 * extend_attention_fwd_unified or decode_attention_fwd call record a HIP
 * event pair on its stream around its attention kernel (for decode, its
 * attention and merge launches); 0 stops recording.
 * pkv_profile_read waits for the recorded events and returns the summed
 * attention-kernel time in milliseconds and the number of calls.  The
 * record is process-wide and holds at most 4096 calls.
 */
int pkv_profile_enable(int on);
int pkv_profile_read(double* total_ms, int64_t* calls);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
