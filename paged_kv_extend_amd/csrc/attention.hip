// Extend attention kernel and split-merge kernel for gfx950.
//
// What is computed follows the SGLang page "extend_attention.py",
// _fwd_kernel_unified: logits are q.k times the scale, optionally soft-capped
// (cap * tanh(s / cap)), masked so that new token i of a sequence with P
// prefix tokens sees keys j <= P + i, and combined with an online softmax
// whose probabilities are rounded to the value dtype before the P.V product.
// The key sequence is the prefix, gathered from the token-granular pool
// through kv_indices, followed by the sequence's own new tokens (page
// "flashinfer_backend.py", forward_extend / call_begin_forward: prefix via
// kv_indptr/kv_indices, new K/V rows addressed by qo_indptr).
//
// Design (MI355X):
//  * One workgroup = 4 waves = 128 packed query rows (token-major packing of
//    the G query heads that share a KV head), one KV tile of BN keys at a
//    time staged in LDS and shared by all 128 rows.
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: K is the A operand read from
//    LDS, Q^T the B operand held in registers.  In the result a lane owns one
//    query row, so the row max and row sum of the online softmax are per-lane
//    values plus one exchange between lanes l and l+32 (v_permlane32_swap).
//  * O^T = V^T . P^T: the probabilities already sit in the B-operand layout
//    (the MFMA contraction index is permuted consistently on both operands),
//    V is stored transposed in LDS so each lane reads two 8-byte runs of
//    keys.  The accumulator rescale by exp2(m_old - m_new) is a per-lane
//    scalar multiply.
//  * Keys are processed as one sequence (prefix then new tokens); tiles past
//    the last visible key of a wave are skipped and only tiles crossing the
//    causal diagonal pay for the mask.
//  * fp32 inputs use v_mfma_f32_32x32x2f32 with the same structure (no
//    rounding of probabilities), so fp32 results carry fp32 products.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value over lanes l and l^32
__device__ __forceinline__ float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Logit in base-2 units: scale * s * log2(e), or cap * tanh(scale * s / cap) * log2(e).
// tanh(y) = 1 - 2 / (e^{2y} + 1) saturates cleanly to +-1 for large |y|.
template <bool CAP>
__device__ __forceinline__ float logit2(float s, const AttnArgs& a) {
  if constexpr (CAP) {
    float e = fast_exp2(s * a.cap_in * (2.0f * kLog2e));
    return a.cap_out * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
  } else {
    return s * a.scale_log2;
  }
}

template <bool F32>
struct Elem;
template <>
struct Elem<false> {
  using T = uint16_t;  // bf16 bit pattern
  static constexpr int kVec = 8;  // elements per 16-byte chunk
};
template <>
struct Elem<true> {
  using T = float;
  static constexpr int kVec = 4;
};

// Row source for key j of sequence (prefix P, new tokens E): >= 0 pool slot,
// -1 zero row (past the sequence), <= -2 encodes new-token row (q0 + j - P) as -(row + 2).
__device__ __forceinline__ int64_t key_source(int j, int P, int E, int q0, int kvs,
                                              const int64_t* __restrict__ kv_indices) {
  if (j < P) return kv_indices[kvs + j];
  if (j < P + E) return -2 - (int64_t)(q0 + j - P);
  return -1;
}

template <bool F32, int LQ, int LV, int BN>
struct Cfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;
  static constexpr int VEC = Elem<F32>::kVec;
  // LDS pitches in elements.  bf16: K row-major [BN][LQ+8] (16-byte reads,
  // 8 consecutive rows hit 8 distinct 4-bank groups); V transposed
  // [LV][BN+4] (8-byte reads, 16 consecutive rows hit distinct bank pairs).
  // fp32: K [BN][LQ+1], V row-major [BN][LV+1].
  static constexpr int KROW = F32 ? LQ + 1 : LQ + 8;
  static constexpr int VROW = F32 ? LV + 1 : BN + 4;
  static constexpr int K_ELEMS = BN * KROW;
  static constexpr int V_ELEMS = F32 ? BN * VROW : LV * VROW;
  static constexpr int K_CHUNKS = BN * LQ / VEC;          // 16-byte chunks per K tile
  static constexpr int K_PER_THREAD = (K_CHUNKS + NT - 1) / NT;
  // bf16 V: blocks of 4 keys x 8 columns; fp32 V: 16-byte chunks like K
  static constexpr int V_UNITS = F32 ? BN * LV / VEC : (BN / 4) * (LV / 8);
  static constexpr int V_PER_THREAD = (V_UNITS + NT - 1) / NT;
  static_assert(BN % 32 == 0 && LQ % 16 == 0 && LV % 32 == 0, "tile shape");
};

template <bool F32, int LQ, int LV, int BN, bool CAP, int MINB>
__global__ __launch_bounds__(256, MINB) void attn_kernel(AttnArgs a) {
  using C = Cfg<F32, LQ, LV, BN>;
  using T = typename Elem<F32>::T;
  constexpr int NT = C::NT, BM = C::BM, VEC = C::VEC;
  constexpr int KROW = C::KROW, VROW = C::VROW;
  constexpr int NKB = BN / 32;  // 32-key blocks per tile
  constexpr int NDB = LV / 32;  // 32-column blocks of the output

  __shared__ __attribute__((aligned(16))) T lds[C::K_ELEMS + C::V_ELEMS];
  T* __restrict__ Ks = lds;
  T* __restrict__ Vs = lds + C::K_ELEMS;

  if ((int)blockIdx.x >= a.hdr->num_work) return;
  const WorkItem it = a.work[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int qi = lane & 31, hi = lane >> 5;
  const int G = a.group;
  const int b = it.b, g = it.g;
  const int q0 = a.qo_indptr[b], E = a.qo_indptr[b + 1] - q0;
  const int kvs = a.kv_indptr[b], P = a.kv_indptr[b + 1] - kvs;
  const int R = E * G;

  // this lane's query row
  const int r = it.t * BM + wv * 32 + qi;
  const bool valid = r < R;
  const int tok = valid ? r / G : 0;
  const int head = g * G + (valid ? r % G : 0);
  const int lim = valid ? P + tok : -1;  // last visible key
  // the wave's token range (rows are token-major)
  const int rw0 = it.t * BM + wv * 32;
  const bool wave_live = rw0 < R;
  const int i_lo_w = wave_live ? rw0 / G : 0;
  const int i_hi_w = wave_live ? min(R - 1, rw0 + 31) / G : 0;

  const T* __restrict__ qp = reinterpret_cast<const T*>(a.q);
  const T* __restrict__ kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* __restrict__ vpool = reinterpret_cast<const T*>(a.v_pool);
  const T* __restrict__ kext = reinterpret_cast<const T*>(a.k_ext);
  const T* __restrict__ vext = reinterpret_cast<const T*>(a.v_ext);

  // ---- Q^T operand in registers
  constexpr int NQ = F32 ? LQ / 2 : LQ / 16;
  using QT = typename std::conditional<F32, float, bf16x8>::type;
  QT qr[NQ];
  {
    const T* qrow = qp + (int64_t)(q0 + tok) * a.q_st + (int64_t)head * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
      if constexpr (F32) {
        qr[ks] = valid ? qrow[2 * ks + hi] : 0.0f;
      } else {
        uint4 v = valid ? *reinterpret_cast<const uint4*>(qrow + ks * 16 + hi * 8) : make_uint4(0, 0, 0, 0);
        qr[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;  // running max, base-2 units
  float l_run = 0.0f;       // this lane's share of the running sum

  // ---- global -> register staging of one KV tile
  uint4 kreg[C::K_PER_THREAD];
  uint4 vreg[C::V_PER_THREAD][F32 ? 1 : 4];

  auto load_tile = [&](int kt) {
    const int j0 = kt * BN;
#pragma unroll
    for (int u = 0; u < C::K_PER_THREAD; ++u) {
      const int c = tid + u * NT;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (C::K_CHUNKS % NT == 0 || c < C::K_CHUNKS) {
        const int row = c / (LQ / VEC), col = (c % (LQ / VEC)) * VEC;
        const int64_t src = key_source(j0 + row, P, E, q0, kvs, a.kv_indices);
        if (src >= 0)
          v = *reinterpret_cast<const uint4*>(kpool + src * a.kp_ss + (int64_t)g * a.kp_sh + col);
        else if (src <= -2)
          v = *reinterpret_cast<const uint4*>(kext + (-2 - src) * a.ke_st + (int64_t)g * a.ke_sh + col);
      }
      kreg[u] = v;
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_THREAD; ++u) {
      const int c = tid + u * NT;
      if constexpr (F32) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (C::V_UNITS % NT == 0 || c < C::V_UNITS) {
          const int row = c / (LV / VEC), col = (c % (LV / VEC)) * VEC;
          const int64_t src = key_source(j0 + row, P, E, q0, kvs, a.kv_indices);
          if (src >= 0)
            v = *reinterpret_cast<const uint4*>(vpool + src * a.vp_ss + (int64_t)g * a.vp_sh + col);
          else if (src <= -2)
            v = *reinterpret_cast<const uint4*>(vext + (-2 - src) * a.ve_st + (int64_t)g * a.ve_sh + col);
        }
        vreg[u][0] = v;
      } else {
        const bool in = C::V_UNITS % NT == 0 || c < C::V_UNITS;
        const int kq = c % (BN / 4), col = (c / (BN / 4)) * 8;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          uint4 v = make_uint4(0, 0, 0, 0);
          if (in) {
            const int64_t src = key_source(j0 + 4 * kq + rr, P, E, q0, kvs, a.kv_indices);
            if (src >= 0)
              v = *reinterpret_cast<const uint4*>(vpool + src * a.vp_ss + (int64_t)g * a.vp_sh + col);
            else if (src <= -2)
              v = *reinterpret_cast<const uint4*>(vext + (-2 - src) * a.ve_st + (int64_t)g * a.ve_sh + col);
          }
          vreg[u][rr] = v;
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < C::K_PER_THREAD; ++u) {
      const int c = tid + u * NT;
      if (C::K_CHUNKS % NT == 0 || c < C::K_CHUNKS) {
        const int row = c / (LQ / VEC), col = (c % (LQ / VEC)) * VEC;
        if constexpr (F32) {
          float* dst = Ks + row * KROW + col;
          dst[0] = __uint_as_float(kreg[u].x);
          dst[1] = __uint_as_float(kreg[u].y);
          dst[2] = __uint_as_float(kreg[u].z);
          dst[3] = __uint_as_float(kreg[u].w);
        } else {
          *reinterpret_cast<uint4*>(Ks + row * KROW + col) = kreg[u];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_THREAD; ++u) {
      const int c = tid + u * NT;
      if (C::V_UNITS % NT == 0 || c < C::V_UNITS) {
        if constexpr (F32) {
          const int row = c / (LV / VEC), col = (c % (LV / VEC)) * VEC;
          float* dst = Vs + row * VROW + col;
          dst[0] = __uint_as_float(vreg[u][0].x);
          dst[1] = __uint_as_float(vreg[u][0].y);
          dst[2] = __uint_as_float(vreg[u][0].z);
          dst[3] = __uint_as_float(vreg[u][0].w);
        } else {
          // transpose 4 keys x 8 columns into 8 rows of V^T, 4 keys (8 bytes) each
          const int kq = c % (BN / 4), col = (c / (BN / 4)) * 8;
          const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&vreg[u][0]);
          const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&vreg[u][1]);
          const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&vreg[u][2]);
          const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&vreg[u][3]);
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            // columns col+2*w2 (low halves) and col+2*w2+1 (high halves)
            uint2 lo, hi2;
            lo.x = __builtin_amdgcn_perm(r1[w2], r0[w2], 0x05040100u);
            lo.y = __builtin_amdgcn_perm(r3[w2], r2[w2], 0x05040100u);
            hi2.x = __builtin_amdgcn_perm(r1[w2], r0[w2], 0x07060302u);
            hi2.y = __builtin_amdgcn_perm(r3[w2], r2[w2], 0x07060302u);
            *reinterpret_cast<uint2*>(Vs + (col + 2 * w2) * VROW + 4 * kq) = lo;
            *reinterpret_cast<uint2*>(Vs + (col + 2 * w2 + 1) * VROW + 4 * kq) = hi2;
          }
        }
      }
    }
  };

  const int kt0 = it.kt_begin, kt1 = it.kt_end;
  if (kt0 < kt1) load_tile(kt0);
  for (int kt = kt0; kt < kt1; ++kt) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (kt + 1 < kt1) load_tile(kt + 1);  // in flight while this tile is computed

    const int j0 = kt * BN;
    if (!wave_live || j0 > P + i_hi_w) continue;  // nothing visible for this wave
    const bool need_mask = j0 + BN - 1 > P + i_lo_w;

    // S^T = K Q^T for the tile's 32-key blocks
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
      const T* krow = Ks + (kb * 32 + qi) * KROW;
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) {
        if constexpr (F32) {
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * ks + hi], qr[ks], s[kb], 0, 0, 0);
        } else {
          bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + ks * 16 + hi * 8));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qr[ks], s[kb], 0, 0, 0);
        }
      }
    }

    // logits (base 2), mask, row max
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float x = logit2<CAP>(s[kb][rr], a);
        if (need_mask) {
          const int j = j0 + kb * 32 + 8 * (rr / 4) + 4 * hi + (rr % 4);
          x = j <= lim ? x : -INFINITY;
        }
        s[kb][rr] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;

    // P and O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if constexpr (F32) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const float p = fast_exp2(s[kb][rr] - m_use);
          l_run += p;
          const int key = kb * 32 + 8 * (rr / 4) + 4 * hi + (rr % 4);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VROW + db * 32 + qi], p, acc[db], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = fast_exp2(s[kb][8 * half + e] - m_use);
            l_run += p;
            pb[e] = (__bf16)p;
          }
          const int kcol = kb * 32 + 16 * half + 4 * hi;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const T* vrow = Vs + (db * 32 + qi) * VROW + kcol;
            uint2 v0 = *reinterpret_cast<const uint2*>(vrow);
            uint2 v1 = *reinterpret_cast<const uint2*>(vrow + 8);
            bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc[db], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- epilogue
  const float l_tot = pair_sum(l_run);
  if (it.part < 0) {
    if (!valid) return;
    const float inv = 1.0f / l_tot;
    T* orow = reinterpret_cast<T*>(a.o) + (int64_t)(q0 + tok) * a.o_st + (int64_t)head * a.o_sh;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hi;
        if constexpr (F32) {
          *reinterpret_cast<float4*>(orow + d) =
              make_float4(acc[db][4 * g4] * inv, acc[db][4 * g4 + 1] * inv, acc[db][4 * g4 + 2] * inv,
                          acc[db][4 * g4 + 3] * inv);
        } else {
          bf16x4 ov;
          ov[0] = (__bf16)(acc[db][4 * g4] * inv);
          ov[1] = (__bf16)(acc[db][4 * g4 + 1] * inv);
          ov[2] = (__bf16)(acc[db][4 * g4 + 2] * inv);
          ov[3] = (__bf16)(acc[db][4 * g4 + 3] * inv);
          *reinterpret_cast<bf16x4*>(orow + d) = ov;
        }
      }
    }
  } else {
    // unnormalised partial state of this chunk, one slot row per packed row
    const int64_t prow = (int64_t)it.part * BM + wv * 32 + qi;
    float* pa = a.part_acc + prow * LV;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hi;
        *reinterpret_cast<float4*>(pa + d) =
            make_float4(acc[db][4 * g4], acc[db][4 * g4 + 1], acc[db][4 * g4 + 2], acc[db][4 * g4 + 3]);
      }
    }
    if (hi == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(m_run, l_tot);
  }
}

// Merge of the chunks of split items, in chunk order (deterministic):
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o = sum_s acc_s 2^(m_s - M) / L
// which is the log-sum-exp state merge (page "flashinfer_backend.py",
// forward_extend, merge_state of the ragged and paged partial outputs).
template <bool F32, int LV>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int bm) {
  using T = typename Elem<F32>::T;
  if ((int)blockIdx.x >= a.hdr->num_merge) return;
  const MergeItem mi = a.merge[blockIdx.x];
  const int G = a.group;
  const int q0 = a.qo_indptr[mi.b], E = a.qo_indptr[mi.b + 1] - q0;
  const int R = E * G;
  constexpr int V4 = LV / 4;
  for (int idx = threadIdx.x; idx < bm * V4; idx += 256) {
    const int row = idx / V4, d = (idx % V4) * 4;
    const int r = mi.t * bm + row;
    if (r >= R) continue;
    float M = -INFINITY;
    for (int s = 0; s < mi.n; ++s) M = fmaxf(M, a.part_ml[((int64_t)(mi.part_base + s) * bm + row) * 2]);
    float L = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < mi.n; ++s) {
      const int64_t prow = (int64_t)(mi.part_base + s) * bm + row;
      const float w = fast_exp2(a.part_ml[prow * 2] - M);
      L += a.part_ml[prow * 2 + 1] * w;
      const float4 v = *reinterpret_cast<const float4*>(a.part_acc + prow * LV + d);
      o.x += v.x * w;
      o.y += v.y * w;
      o.z += v.z * w;
      o.w += v.w * w;
    }
    const float inv = 1.0f / L;
    const int tok = r / G, head = mi.g * G + r % G;
    T* orow = reinterpret_cast<T*>(a.o) + (int64_t)(q0 + tok) * a.o_st + (int64_t)head * a.o_sh + d;
    if constexpr (F32) {
      *reinterpret_cast<float4*>(orow) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    } else {
      bf16x4 ov;
      ov[0] = (__bf16)(o.x * inv);
      ov[1] = (__bf16)(o.y * inv);
      ov[2] = (__bf16)(o.z * inv);
      ov[3] = (__bf16)(o.w * inv);
      *reinterpret_cast<bf16x4*>(orow) = ov;
    }
  }
}

template <bool F32, int LQ, int LV, int BN, int MINB>
hipError_t launch_attn_t(const AttnArgs& a, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (a.use_cap)
    hipLaunchKernelGGL((attn_kernel<F32, LQ, LV, BN, true, MINB>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<F32, LQ, LV, BN, false, MINB>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <bool F32, int LQ, int LV, int BN, int MINB>
int occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_kernel<F32, LQ, LV, BN, false, MINB>, 256, 0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

// The supported (dtype, lq, lv) variants and their key-tile widths.
#define PKV_VARIANTS(X)          \
  X(false, 64, 64, 64, 2)        \
  X(false, 128, 128, 64, 2)      \
  X(false, 256, 256, 32, 1)      \
  X(false, 192, 128, 32, 2)      \
  X(false, 288, 256, 32, 1)      \
  X(false, 576, 512, 32, 1)      \
  X(true, 64, 64, 32, 1)         \
  X(true, 128, 128, 32, 1)

}  // namespace

bool attn_tiling(int dtype, int lq, int lv, Tiling* t) {
  const bool f32 = dtype == 1;
#define PKV_TILING(F, Q, V, N, M)              \
  if (f32 == F && lq == Q && lv == V) {        \
    t->bm = 128;                               \
    t->bn = N;                                 \
    t->threads = 256;                          \
    return true;                               \
  }
  PKV_VARIANTS(PKV_TILING)
#undef PKV_TILING
  return false;
}

hipError_t launch_attention(int dtype, int lq, int lv, const AttnArgs& a, int64_t grid, hipStream_t s) {
  const bool f32 = dtype == 1;
#define PKV_LAUNCH(F, Q, V, N, M) \
  if (f32 == F && lq == Q && lv == V) return launch_attn_t<F, Q, V, N, M>(a, grid, s);
  PKV_VARIANTS(PKV_LAUNCH)
#undef PKV_LAUNCH
  return hipErrorInvalidValue;
}

int attention_blocks_per_cu(int dtype, int lq, int lv) {
  const bool f32 = dtype == 1;
#define PKV_OCC(F, Q, V, N, M) \
  if (f32 == F && lq == Q && lv == V) return occupancy_t<F, Q, V, N, M>();
  PKV_VARIANTS(PKV_OCC)
#undef PKV_OCC
  return 1;
}

hipError_t launch_merge(int dtype, int lv, const AttnArgs& a, int bm, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const bool f32 = dtype == 1;
#define PKV_MERGE(F, V)                                                                             \
  if (f32 == F && lv == V) {                                                                        \
    hipLaunchKernelGGL((merge_kernel<F, V>), dim3((unsigned)grid), dim3(256), 0, s, a, bm);          \
    return hipGetLastError();                                                                       \
  }
  PKV_MERGE(false, 64)
  PKV_MERGE(false, 128)
  PKV_MERGE(false, 256)
  PKV_MERGE(false, 512)
  PKV_MERGE(true, 64)
  PKV_MERGE(true, 128)
#undef PKV_MERGE
  return hipErrorInvalidValue;
}

}  // namespace pkv
