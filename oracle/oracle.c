/*
 * CPU oracle for paged-KV extend attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this library.  It shares no code, header or table with the HIP library and
 * is written for obviousness, not speed: plain loops, double accumulation.
 *
 * Sources (the SGLang pages on extend attention):
 *  - unified index build: page "extend_attention.py" (sglang 0.5.3rc2 ->
 *    0.5.4.post1 diff), functions build_unified_kv_indices and
 *    _copy_unified_indices_kernel;
 *  - attention: the same page, kernel _fwd_kernel_unified (causal mask, scale,
 *    soft-cap, softmax; and, for the unified entry, keys read through one
 *    index array) and the reference helper redundant_attention
 *    (attention over the concatenated prefix + extend sequence, keeping the
 *    extend rows); page "flashinfer_backend.py", forward_extend and
 *    call_begin_forward (the prefix is read through kv_indptr/kv_indices,
 *    the new tokens' K/V share qo_indptr with the queries).
 *
 *  - decode attention: page "flashinfer_backend.py", forward_decode and the
 *    decode index updater (one query token per request over its pool keys,
 *    with the sliding-window key range of update_sliding_window).
 *
 *  - the steps before attention: the KV-cache store of the new tokens
 *    (page "flashinfer_backend.py", forward_extend, set_kv_buffer) and the
 *    prefix index gather from the request-to-token table (the same page,
 *    create_flashinfer_kv_indices_triton).
 *
 * Parity of every function is pinned by tests/test_oracle_pins.py (worked
 * examples, library routines, closed forms and invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)
#define ORACLE_ERANGE (-3)

/*
 * Unified KV index build (extend_attention.py, build_unified_kv_indices and
 * _copy_unified_indices_kernel).  For every sequence b:
 *   prefix_lens[b] = prefix_kv_indptr[b+1] - prefix_kv_indptr[b]
 *   unified_kv_indptr = [0, running sum of prefix_lens[b] + extend_seq_lens[b]]
 *   unified segment b = prefix_kv_indices[prefix_kv_indptr[b] ...] (prefix_lens[b] entries)
 *                       followed by extend_kv_indices[extend_start_loc[b] ...]
 *                       (extend_seq_lens[b] entries).
 * Only the first bs entries of extend_start_loc / extend_seq_lens are read.
 */
int oracle_build_unified_kv_indices(const int32_t* prefix_kv_indptr,
                                    const int64_t* prefix_kv_indices,
                                    const int32_t* extend_start_loc,
                                    const int32_t* extend_seq_lens,
                                    const int64_t* extend_kv_indices, int32_t bs,
                                    int32_t* unified_kv_indptr, int64_t* unified_kv_indices,
                                    int32_t* prefix_lens) {
  if (bs < 0) return ORACLE_EINVAL;
  int64_t running = 0;
  unified_kv_indptr[0] = 0;
  for (int32_t b = 0; b < bs; ++b) {
    int32_t p_start = prefix_kv_indptr[b];
    int32_t p_len = prefix_kv_indptr[b + 1] - prefix_kv_indptr[b];
    int32_t e_start = extend_start_loc[b];
    int32_t e_len = extend_seq_lens[b];
    if (p_len < 0 || e_len < 0) return ORACLE_EINVAL;
    if (prefix_lens) prefix_lens[b] = p_len;
    int64_t u = running;
    for (int32_t o = 0; o < p_len; ++o) unified_kv_indices[u + o] = prefix_kv_indices[p_start + o];
    for (int32_t o = 0; o < e_len; ++o)
      unified_kv_indices[u + p_len + o] = extend_kv_indices[e_start + o];
    running += (int64_t)p_len + (int64_t)e_len;
    unified_kv_indptr[b + 1] = (int32_t)running;
  }
  return ORACLE_OK;
}

/* Element access: dtype 0 = bf16 bit patterns (uint16), 1 = float32. */
static inline double load_elem(const void* base, int dtype, int64_t off) {
  if (dtype == 1) return (double)((const float*)base)[off];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[off]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Sequence that owns extend-token row t: the b with qo_indptr[b] <= t < qo_indptr[b+1]. */
static int32_t owner_seq(const int32_t* qo_indptr, int32_t bs, int64_t t) {
  for (int32_t b = 0; b < bs; ++b)
    if (t >= qo_indptr[b] && t < qo_indptr[b + 1]) return b;
  return -1;
}

/*
 * Extend attention, one output row per (extend token t, query head h).
 *
 * Sequence b owns t; i = t - qo_indptr[b] is the query's position among the
 * b's new tokens; P = prefix length, g = h / (hq / hkv) its KV head.  The key
 * sequence is the concatenation of the prefix (key j < P comes from pool slot
 * kv_indices[kv_indptr[b] + j]) and the new tokens (key j >= P is row
 * qo_indptr[b] + j - P of k_ext / v_ext).  Query i sees key j iff j <= P + i:
 * the whole prefix, and the new tokens up to and including itself.
 *   s_j = scale * <q, K_j>; with a cap c > 0, s_j = c * tanh(s_j / c)
 *   out = sum_j exp(s_j - max s) V_j / (sum_j exp(s_j - max s) + sink term)
 * scale = sm_scale, or 1/sqrt(lq) when sm_scale == 0.
 * Options of _fwd_kernel_unified (extend_attention.py): a sliding window
 * W > 0 also hides keys j < P + i - W (the query's absolute position may be
 * at most W past the key's); sinks (NULL: none) add exp(sinks[h] - max s) to
 * the denominator of query head h; a custom mask (NULL: none) replaces the
 * causal rule: with L = P + E keys, query i sees key j < L iff
 * custom_mask[mask_indptr[b] + i * L + j] != 0 (a byte matrix per sequence).
 */
int oracle_extend_attention(int32_t dtype,
                            const void* q, int64_t q_st, int64_t q_sh,
                            const void* k_ext, int64_t ke_st, int64_t ke_sh,
                            const void* v_ext, int64_t ve_st, int64_t ve_sh,
                            const void* k_pool, int64_t kp_ss, int64_t kp_sh,
                            const void* v_pool, int64_t vp_ss, int64_t vp_sh,
                            int64_t pool_slots,
                            const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int64_t* kv_indices,
                            int32_t bs, int32_t hq, int32_t hkv, int32_t lq, int32_t lv,
                            double sm_scale, double logit_cap,
                            const int64_t* rows, int64_t n_rows,
                            double* out, int32_t num_threads, int32_t window, const float* sinks,
                            const uint8_t* custom_mask, const int64_t* mask_indptr) {
  if (bs < 0 || hq <= 0 || hkv <= 0 || lq <= 0 || lv <= 0) return ORACLE_EINVAL;
  if (hq % hkv != 0 || (dtype != 0 && dtype != 1)) return ORACLE_EINVAL;
  const int32_t group = hq / hkv;
  const int64_t total_q = bs > 0 ? qo_indptr[bs] : 0;
  const double scale = sm_scale != 0.0 ? sm_scale : 1.0 / sqrt((double)lq);
  if (rows == NULL) n_rows = total_q;

  int64_t max_keys = 1;
  for (int32_t b = 0; b < bs; ++b) {
    int64_t keys = (int64_t)(kv_indptr[b + 1] - kv_indptr[b]) + (qo_indptr[b + 1] - qo_indptr[b]);
    if (keys > max_keys) max_keys = keys;
  }
  for (int64_t n = 0; n < kv_indptr[bs] - kv_indptr[0]; ++n) {
    int64_t slot = kv_indices[kv_indptr[0] + n];
    if (slot < 0 || slot >= pool_slots) return ORACLE_ERANGE;
  }

  int status = ORACLE_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)max_keys);
    char* vis = (char*)malloc((size_t)max_keys);
    double* acc = (double*)malloc(sizeof(double) * (size_t)lv);
    if (!s || !vis || !acc) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t w = 0; w < n_rows * hq; ++w) {
        int64_t r = w / hq;
        int32_t h = (int32_t)(w % hq);
        int64_t t = rows ? rows[r] : r;
        int32_t b = owner_seq(qo_indptr, bs, t);
        double* o = out + (r * hq + h) * (int64_t)lv;
        if (b < 0) {
#pragma omp atomic write
          status = ORACLE_EINVAL;
          continue;
        }
        int64_t i = t - qo_indptr[b];
        int64_t P = kv_indptr[b + 1] - kv_indptr[b];
        int32_t g = h / group;
        int64_t E = qo_indptr[b + 1] - qo_indptr[b];
        /* visible keys: causal (j <= P + i) or the custom mask, then the window */
        int64_t visible = custom_mask ? P + E : P + i + 1;
        int64_t first = (window > 0 && P + i - window > 0) ? P + i - window : 0;
        for (int64_t j = first; j < visible; ++j)
          vis[j] = custom_mask ? custom_mask[mask_indptr[b] + i * (P + E) + j] != 0 : 1;

        /* logits of the visible keys */
        double m = -INFINITY;
        for (int64_t j = first; j < visible; ++j) {
          if (!vis[j]) continue;
          const void* kbase;
          int64_t koff;
          if (j < P) {
            kbase = k_pool;
            koff = kv_indices[kv_indptr[b] + j] * kp_ss + (int64_t)g * kp_sh;
          } else {
            kbase = k_ext;
            koff = (qo_indptr[b] + (j - P)) * ke_st + (int64_t)g * ke_sh;
          }
          double dot = 0.0;
          for (int32_t d = 0; d < lq; ++d)
            dot += load_elem(q, dtype, t * q_st + (int64_t)h * q_sh + d) *
                   load_elem(kbase, dtype, koff + d);
          double x = dot * scale;
          if (logit_cap > 0.0) x = logit_cap * tanh(x / logit_cap);
          s[j] = x;
          if (x > m) m = x;
        }

        /* softmax-weighted sum of the visible values */
        double den = 0.0;
        for (int32_t d = 0; d < lv; ++d) acc[d] = 0.0;
        for (int64_t j = first; j < visible; ++j) {
          if (!vis[j]) continue;
          const void* vbase;
          int64_t voff;
          if (j < P) {
            vbase = v_pool;
            voff = kv_indices[kv_indptr[b] + j] * vp_ss + (int64_t)g * vp_sh;
          } else {
            vbase = v_ext;
            voff = (qo_indptr[b] + (j - P)) * ve_st + (int64_t)g * ve_sh;
          }
          double wgt = exp(s[j] - m);
          den += wgt;
          for (int32_t d = 0; d < lv; ++d) acc[d] += wgt * load_elem(vbase, dtype, voff + d);
        }
        if (sinks) den += exp((double)sinks[h] - m);
        for (int32_t d = 0; d < lv; ++d) o[d] = den > 0.0 ? acc[d] / den : NAN;
      }
    }
    free(s);
    free(vis);
    free(acc);
  }
  return status;
}

/*
 * Unified one-stage extend attention (extend_attention.py,
 * extend_attention_fwd_unified and _fwd_kernel_unified): every key of a
 * sequence, prefix and new tokens alike, is read from the pool through one
 * index array.
 *
 * Sequence b owns extend-token row t, i = t - qo_indptr[b].  Its keys are
 * j = 0 .. L-1 with L = kv_indptr[b+1] - kv_indptr[b]; key j is pool slot
 * kv_indices[kv_indptr[b] + j].  With P = prefix_lens[b], key j is visible to
 * query i iff j < P (a prefix key) or j - P <= i (a new token at or before the
 * query).  Scale, cap, softmax, window and sinks as in
 * oracle_extend_attention (the window also hides j < P + i - W); a custom
 * mask replaces the causal rule: key j < L is seen iff
 * custom_mask[mask_indptr[b] + i * L + j] != 0.  A row with no visible key
 * and no sink gets NaN (the denominator is zero).
 */
int oracle_extend_attention_unified(int32_t dtype,
                                    const void* q, int64_t q_st, int64_t q_sh,
                                    const void* k_pool, int64_t kp_ss, int64_t kp_sh,
                                    const void* v_pool, int64_t vp_ss, int64_t vp_sh,
                                    int64_t pool_slots,
                                    const int32_t* qo_indptr, const int32_t* kv_indptr,
                                    const int64_t* kv_indices, const int32_t* prefix_lens,
                                    int32_t bs, int32_t hq, int32_t hkv, int32_t lq, int32_t lv,
                                    double sm_scale, double logit_cap,
                                    const int64_t* rows, int64_t n_rows,
                                    double* out, int32_t num_threads, int32_t window, const float* sinks,
                                    const uint8_t* custom_mask, const int64_t* mask_indptr) {
  if (bs < 0 || hq <= 0 || hkv <= 0 || lq <= 0 || lv <= 0) return ORACLE_EINVAL;
  if (hq % hkv != 0 || (dtype != 0 && dtype != 1)) return ORACLE_EINVAL;
  const int32_t group = hq / hkv;
  const int64_t total_q = bs > 0 ? qo_indptr[bs] : 0;
  const double scale = sm_scale != 0.0 ? sm_scale : 1.0 / sqrt((double)lq);
  if (rows == NULL) n_rows = total_q;

  int64_t max_keys = 1;
  for (int32_t b = 0; b < bs; ++b) {
    int64_t keys = (int64_t)(kv_indptr[b + 1] - kv_indptr[b]);
    if (keys > max_keys) max_keys = keys;
  }
  for (int64_t n = 0; n < kv_indptr[bs] - kv_indptr[0]; ++n) {
    int64_t slot = kv_indices[kv_indptr[0] + n];
    if (slot < 0 || slot >= pool_slots) return ORACLE_ERANGE;
  }

  int status = ORACLE_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)max_keys);
    char* seen = (char*)malloc((size_t)max_keys);
    double* acc = (double*)malloc(sizeof(double) * (size_t)lv);
    if (!s || !seen || !acc) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t w = 0; w < n_rows * hq; ++w) {
        int64_t r = w / hq;
        int32_t h = (int32_t)(w % hq);
        int64_t t = rows ? rows[r] : r;
        int32_t b = owner_seq(qo_indptr, bs, t);
        double* o = out + (r * hq + h) * (int64_t)lv;
        if (b < 0) {
#pragma omp atomic write
          status = ORACLE_EINVAL;
          continue;
        }
        int64_t i = t - qo_indptr[b];
        int64_t L = kv_indptr[b + 1] - kv_indptr[b];
        int64_t P = prefix_lens[b];
        int32_t g = h / group;

        /* logits of the visible keys */
        double m = -INFINITY;
        for (int64_t j = 0; j < L; ++j) {
          seen[j] = (custom_mask ? custom_mask[mask_indptr[b] + i * L + j] != 0 : ((j < P) || (j - P <= i))) &&
                    (window <= 0 || j >= P + i - window);
          if (!seen[j]) continue;
          int64_t koff = kv_indices[kv_indptr[b] + j] * kp_ss + (int64_t)g * kp_sh;
          double dot = 0.0;
          for (int32_t d = 0; d < lq; ++d)
            dot += load_elem(q, dtype, t * q_st + (int64_t)h * q_sh + d) * load_elem(k_pool, dtype, koff + d);
          double x = dot * scale;
          if (logit_cap > 0.0) x = logit_cap * tanh(x / logit_cap);
          s[j] = x;
          if (x > m) m = x;
        }

        /* softmax-weighted sum of the visible values */
        double den = 0.0;
        for (int32_t d = 0; d < lv; ++d) acc[d] = 0.0;
        for (int64_t j = 0; j < L; ++j) {
          if (!seen[j]) continue;
          int64_t voff = kv_indices[kv_indptr[b] + j] * vp_ss + (int64_t)g * vp_sh;
          double wgt = exp(s[j] - m);
          den += wgt;
          for (int32_t d = 0; d < lv; ++d) acc[d] += wgt * load_elem(v_pool, dtype, voff + d);
        }
        if (sinks) den += exp((double)sinks[h] - m);
        for (int32_t d = 0; d < lv; ++d) o[d] = den > 0.0 ? acc[d] / den : NAN;
      }
    }
    free(s);
    free(seen);
    free(acc);
  }
  return status;
}

/*
 * Decode attention (flashinfer_backend.py, forward_decode; the decode index
 * updater's update_single_wrapper and update_sliding_window): one query
 * token per request, whose K/V the caller has already stored in the pool,
 * attends to every key of its request, read through kv_indices.
 *
 * Request b has n = kv_indptr[b+1] - kv_indptr[b] keys, key j being pool slot
 * kv_indices[kv_indptr[b] + j]; its query is row b of q.  With a sliding
 * window W > 0 only the last min(n, W + 1) keys are kept (keys j >= n - 1 - W),
 * as the sliding-window updater shortens paged_kernel_lens and moves
 * kv_start_idx.  Scale, cap and softmax as in oracle_extend_attention; a sink
 * adds exp(sink - m) to the denominator.  A request with no key gets zeros.
 *
 * seqs (n_seqs entries, or NULL for all bs requests) selects the requests
 * computed; out is [n_seqs][hq][lv] in double.
 */
int oracle_decode_attention(int32_t dtype,
                            const void* q, int64_t q_st, int64_t q_sh,
                            const void* k_pool, int64_t kp_ss, int64_t kp_sh,
                            const void* v_pool, int64_t vp_ss, int64_t vp_sh,
                            int64_t pool_slots, const int32_t* kv_indptr, const int64_t* kv_indices,
                            int32_t bs, int32_t hq, int32_t hkv, int32_t lq, int32_t lv,
                            double sm_scale, double logit_cap, const int32_t* seqs, int32_t n_seqs,
                            double* out, int32_t num_threads, int32_t window, const float* sinks) {
  if (bs < 0 || hq <= 0 || hkv <= 0 || lq <= 0 || lv <= 0) return ORACLE_EINVAL;
  if (hq % hkv != 0 || (dtype != 0 && dtype != 1)) return ORACLE_EINVAL;
  if (seqs == NULL) n_seqs = bs;
  const int32_t group = hq / hkv;
  const double scale = sm_scale != 0.0 ? sm_scale : 1.0 / sqrt((double)lq);

  int64_t max_keys = 1;
  for (int32_t r = 0; r < n_seqs; ++r) {
    int32_t b = seqs ? seqs[r] : r;
    if (b < 0 || b >= bs) return ORACLE_EINVAL;
    int64_t n = (int64_t)(kv_indptr[b + 1] - kv_indptr[b]);
    if (n > max_keys) max_keys = n;
    for (int64_t j = 0; j < n; ++j) {
      int64_t slot = kv_indices[kv_indptr[b] + j];
      if (slot < 0 || slot >= pool_slots) return ORACLE_ERANGE;
    }
  }

  int status = ORACLE_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel
  {
    double* logit = (double*)malloc(sizeof(double) * (size_t)max_keys);
    double* acc = (double*)malloc(sizeof(double) * (size_t)lv);
    if (!logit || !acc) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t w = 0; w < (int64_t)n_seqs * hq; ++w) {
        int32_t r = (int32_t)(w / hq);
        int32_t h = (int32_t)(w % hq);
        int32_t b = seqs ? seqs[r] : r;
        int32_t g = h / group;
        int64_t n = kv_indptr[b + 1] - kv_indptr[b];
        int64_t first = (window > 0 && n - 1 - window > 0) ? n - 1 - window : 0;
        double* o = out + ((int64_t)r * hq + h) * (int64_t)lv;

        double m = -INFINITY;
        for (int64_t j = first; j < n; ++j) {
          int64_t koff = kv_indices[kv_indptr[b] + j] * kp_ss + (int64_t)g * kp_sh;
          double dot = 0.0;
          for (int32_t d = 0; d < lq; ++d)
            dot += load_elem(q, dtype, (int64_t)b * q_st + (int64_t)h * q_sh + d) * load_elem(k_pool, dtype, koff + d);
          double x = dot * scale;
          if (logit_cap > 0.0) x = logit_cap * tanh(x / logit_cap);
          logit[j] = x;
          if (x > m) m = x;
        }
        for (int32_t d = 0; d < lv; ++d) acc[d] = 0.0;
        if (first >= n) {
          for (int32_t d = 0; d < lv; ++d) o[d] = 0.0;
          continue;
        }
        double den = 0.0;
        for (int64_t j = first; j < n; ++j) {
          int64_t voff = kv_indices[kv_indptr[b] + j] * vp_ss + (int64_t)g * vp_sh;
          double e = exp(logit[j] - m);
          den += e;
          for (int32_t d = 0; d < lv; ++d) acc[d] += e * load_elem(v_pool, dtype, voff + d);
        }
        if (sinks) den += exp((double)sinks[h] - m);
        for (int32_t d = 0; d < lv; ++d) o[d] = acc[d] / den;
      }
    }
    free(logit);
    free(acc);
  }
  return status;
}

/*
 * KV-cache store of the new tokens (flashinfer_backend.py, forward_extend:
 * set_kv_buffer(layer, cache_loc, k, v) before attention reads the pool):
 *   k_pool[out_cache_loc[t], g, :lq] = k_ext[t, g, :lq]
 *   v_pool[out_cache_loc[t], g, :lv] = v_ext[t, g, :lv]
 * for every token t < n_tokens and KV head g; other slots are left alone.
 * Elements are copied as raw bytes of elem_bytes each.  Slots out of
 * [0, pool_slots) are an error (nothing is written then).
 */
int oracle_store_kv_cache(int32_t elem_bytes, int64_t n_tokens, int32_t hkv, int32_t lq, int32_t lv,
                          const void* k_ext, int64_t ke_st, int64_t ke_sh,
                          const void* v_ext, int64_t ve_st, int64_t ve_sh,
                          void* k_pool, int64_t kp_ss, int64_t kp_sh,
                          void* v_pool, int64_t vp_ss, int64_t vp_sh,
                          int64_t pool_slots, const int64_t* out_cache_loc) {
  if (n_tokens < 0 || hkv <= 0 || lq < 0 || lv < 0 || (elem_bytes != 2 && elem_bytes != 4)) return ORACLE_EINVAL;
  for (int64_t t = 0; t < n_tokens; ++t)
    if (out_cache_loc[t] < 0 || out_cache_loc[t] >= pool_slots) return ORACLE_ERANGE;
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t slot = out_cache_loc[t];
    for (int32_t g = 0; g < hkv; ++g) {
      memcpy((char*)k_pool + (slot * kp_ss + (int64_t)g * kp_sh) * elem_bytes,
             (const char*)k_ext + (t * ke_st + (int64_t)g * ke_sh) * elem_bytes, (size_t)lq * elem_bytes);
      memcpy((char*)v_pool + (slot * vp_ss + (int64_t)g * vp_sh) * elem_bytes,
             (const char*)v_ext + (t * ve_st + (int64_t)g * ve_sh) * elem_bytes, (size_t)lv * elem_bytes);
    }
  }
  return ORACLE_OK;
}

/*
 * Prefix index gather from the request-to-token table
 * (flashinfer_backend.py, create_flashinfer_kv_indices_triton and the
 * kv_indptr running sum of call_begin_forward):
 *   kv_indptr[0] = 0, kv_indptr[b+1] = kv_indptr[b] + kv_lens[b]
 *   kv_indices[kv_indptr[b] + o] = req_to_token[req_pool_indices[b] * stride + start_b + o]
 * for o < kv_lens[b], start_b = kv_start_idx[b] (0 when kv_start_idx is NULL).
 * req_to_token holds int32 slots; kv_indices are written as int64.
 */
int oracle_gather_kv_indices(const int32_t* req_to_token, int64_t stride, const int64_t* req_pool_indices,
                             const int32_t* kv_lens, const int32_t* kv_start_idx, int32_t bs,
                             int32_t* kv_indptr, int64_t* kv_indices) {
  if (bs < 0 || stride < 0) return ORACLE_EINVAL;
  kv_indptr[0] = 0;
  for (int32_t b = 0; b < bs; ++b) {
    if (kv_lens[b] < 0) return ORACLE_EINVAL;
    kv_indptr[b + 1] = kv_indptr[b] + kv_lens[b];
  }
  for (int32_t b = 0; b < bs; ++b) {
    int64_t start = kv_start_idx ? kv_start_idx[b] : 0;
    for (int32_t o = 0; o < kv_lens[b]; ++o)
      kv_indices[kv_indptr[b] + o] = (int64_t)req_to_token[req_pool_indices[b] * stride + start + o];
  }
  return ORACLE_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
