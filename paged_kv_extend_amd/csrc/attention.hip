// Extend attention kernel and split-merge kernel for gfx950.
//
// What is computed follows the SGLang page "extend_attention.py",
// _fwd_kernel_unified: logits are q.k times the scale, optionally soft-capped
// (cap * tanh(s / cap)), masked so that new token i of a sequence with P
// prefix tokens sees keys j <= P + i, and combined with an online softmax
// whose probabilities are rounded to the value dtype before the P.V product
// (here the row sum adds the same rounded probabilities).
// The key sequence is the prefix, gathered from the token-granular pool
// through kv_indices, followed by the sequence's own new tokens (page
// "flashinfer_backend.py", forward_extend / call_begin_forward: prefix via
// kv_indptr/kv_indices, new K/V rows addressed by qo_indptr).
//
// Design (MI355X):
//  * One workgroup = 4 waves = 128 packed query rows (token-major packing of
//    the G query heads that share a KV head), one tile of BN keys at a time
//    staged in LDS and shared by all 128 rows.
//  * Row gather: for every tile a table of BN row pointers (pool slot, new
//    token row, or a zero row past the last key the tile's rows can see) is
//    built in LDS one tile ahead, from index loads issued before the previous
//    tile's math, so the slot lookups never stall the loads.  K and V rows are
//    then fetched with 16-byte lane loads, 16 lanes per 256-byte row, into
//    registers while the current tile is computed, and stored row-major.
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: K is the A operand read from
//    LDS, Q^T the B operand held in registers.  In the result a lane owns one
//    query row, so the row max and row sum of the online softmax are per-lane
//    values plus one exchange between lanes l and l+32 (v_permlane32_swap).
//  * O^T = V^T . P^T: the probabilities already sit in the B-operand layout
//    (the MFMA contraction index is permuted consistently on both operands);
//    the V^T operand comes from the row-major V tile through gfx950's
//    transposing LDS read (ds_read_b64_tr_b16), 4 consecutive keys per lane.
//  * Probabilities are exp2(s * c - m) with the scale folded into one FMA; the
//    reference max m is only raised (and the accumulator rescaled) when a row
//    max exceeds it by more than 2^8, so most tiles skip the rescale.
//  * Tiles past the last visible key of a wave are skipped and only tiles
//    crossing the causal diagonal pay for the mask.
//  * fp32 inputs use v_mfma_f32_32x32x2f32 with the same structure (no
//    rounding of probabilities), so fp32 results carry fp32 products.
#include <type_traits>

#include "merge_tile.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes, kept in registers
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // base-2 headroom before the reference max is raised

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

// global-memory (address space 1) views: loads through them become global_load
template <class T>
using gptr = const __attribute__((address_space(1))) T*;

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

template <bool F32, int LQ, int LV, int BN>
struct Cfg {
  static constexpr int NT = 256;
  static constexpr int BM = 128;
  static constexpr int VEC = Elem<F32>::kVec;
  // LDS pitches in elements, chosen from measured bank-conflict counts on
  // gfx950.  bf16 K [BN][LQ+8]: the 16-byte operand reads of 32 rows are
  // conflict-free when the row pitch is 4 x (odd) dwords modulo 64.  bf16 V
  // [BN][LV+32]: the transposing reads (4 rows x 32 bytes per 16 lanes, two
  // such groups per half-wave) are conflict-free when the pitch is 16 dwords
  // modulo 64.  fp32: one pad element per row.
  static constexpr int KROW = F32 ? LQ + 1 : LQ + 8;
  static constexpr int VROW = F32 ? LV + 1 : LV + 32;
  static constexpr int K_ELEMS = BN * KROW;
  static constexpr int V_ELEMS = BN * VROW;
  static constexpr int KC = BN * LQ / VEC;  // 16-byte chunks per tile
  static constexpr int VC = BN * LV / VEC;
  static constexpr int K_PER_THREAD = (KC + NT - 1) / NT;
  static constexpr int V_PER_THREAD = (VC + NT - 1) / NT;
  static_assert(BN % 32 == 0 && BN <= 64 && LQ % 16 == 0 && LV % 32 == 0, "tile shape");
};

// OPT: a sliding window or a custom mask (which replaces the causal rule) may
// be set -- a variant of its own
template <bool F32, int LQ, int LV, int BN, bool CAP, bool OPT, int MINB>
__global__ __launch_bounds__(256, MINB) void attn_kernel(AttnArgs a) {
  using C = Cfg<F32, LQ, LV, BN>;
  using T = typename Elem<F32>::T;
  constexpr int NT = C::NT, BM = C::BM, VEC = C::VEC;
  constexpr int KROW = C::KROW, VROW = C::VROW;
  constexpr int NKB = BN / 32;  // 32-key blocks per tile
  constexpr int NDB = LV / 32;  // 32-column blocks of the output

  __shared__ __attribute__((aligned(16))) T lds[C::K_ELEMS + C::V_ELEMS];
  __shared__ gptr<T> kptr[2][BN];
  __shared__ gptr<T> vptr[2][BN];
  T* __restrict__ Ks = lds;
  T* __restrict__ Vs = lds + C::K_ELEMS;

  // the work record and the plan header in one round trip: the grid is the
  // workspace's capacity of records, so every block index names a record.
  // (Left alone, the compiler loads each piece right before its first use,
  // one round trip after another; the empty asm takes a field of every 16
  // bytes and the header before the branch.)
  const WorkItem it = a.work[blockIdx.x];
  const int num_work = a.hdr->num_work;
  asm volatile("" ::"s"(it.b), "s"(it.kt_end), "s"(it.q0), "s"(it.n_idx), "s"(num_work));
  if (it.b < 0 || (int)blockIdx.x >= num_work) return;  // empty or unused placement slot
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int qi = lane & 31, hi = lane >> 5;
  const int G = a.group;
  const int b = it.b, g = it.g;
  const bool causal = !OPT || a.custom_mask == nullptr;
  const SeqKeys sk = item_keys(it);
  // last visible key of a row of token i: the diagonal, or every key with a custom mask
  auto last_key = [&](int i) __attribute__((always_inline)) {
    return causal ? min(sk.P + i, sk.n_keys - 1) : sk.n_keys - 1;
  };
  const int q0 = sk.q0, E = sk.E, kvs = sk.kvs, P = sk.P;
  const int R = E * G;

  // this lane's query row
  const int r = it.t * BM + wv * 32 + qi;
  const bool valid = r < R;
  const int tok = valid ? r / G : 0;
  const int head = g * G + (valid ? r % G : 0);
  const int W = OPT ? a.window : 0;
  const int lim = valid ? last_key(tok) : -1;  // last visible key
  const int lo = (W > 0 && valid) ? P + tok - W : kNoLowerKey;  // first visible key (sliding window)
  // the wave's token range (rows are token-major) and the workgroup's last visible key
  const int rw0 = it.t * BM + wv * 32;
  const bool wave_live = rw0 < R;
  const int tok_lo_w = wave_live ? rw0 / G : 0, tok_hi_w = wave_live ? min(R - 1, rw0 + 31) / G : 0;
  const int lim_lo_w = last_key(tok_lo_w);
  const int lim_hi_w = last_key(tok_hi_w);
  const int lo_lo_w = W > 0 ? P + tok_lo_w - W : kNoLowerKey;
  const int lo_hi_w = W > 0 ? P + tok_hi_w - W : kNoLowerKey;
  const int key_last = last_key(min(R - 1, it.t * BM + BM - 1) / G);

  const gptr<T> kpool = (gptr<T>)a.k_pool;
  const gptr<T> vpool = (gptr<T>)a.v_pool;
  const gptr<T> kext = (gptr<T>)a.k_ext;
  const gptr<T> vext = (gptr<T>)a.v_ext;
  const gptr<T> zrow = (gptr<T>)a.zero_row;

  // ---- Q^T operand in registers (negated when the scale is negative)
  constexpr int NQ = F32 ? LQ / 2 : LQ / 16;
  using QT = typename std::conditional<F32, float, bf16x8>::type;
  QT qr[NQ];
  {
    const T* qrow = reinterpret_cast<const T*>(a.q) + (int64_t)(q0 + tok) * a.q_st + (int64_t)head * a.q_sh;
    const uint32_t flip = a.neg_q ? (F32 ? 0x80000000u : 0x80008000u) : 0u;
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
      if constexpr (F32) {
        qr[ks] = valid ? __uint_as_float(__float_as_uint(qrow[2 * ks + hi]) ^ flip) : 0.0f;
      } else {
        uint4 v = valid ? *reinterpret_cast<const uint4*>(qrow + ks * 16 + hi * 8) : make_uint4(0, 0, 0, 0);
        v.x ^= flip;
        v.y ^= flip;
        v.z ^= flip;
        v.w ^= flip;
        qr[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_ref = -INFINITY;  // reference max of the exponentials, base-2 units
  float l_run = 0.0f;       // this lane's share of the running sum

  // ---- row pointer tables: thread t < BN owns key kt*BN + t
  const int kt0 = it.kt_begin, kt1 = it.kt_end;
  int64_t slot_next = 0;  // prefetched pool slot for the key this thread owns two tiles ahead
  auto fetch_slot = [&](int kt) __attribute__((always_inline)) {
    const int j = kt * BN + tid;
    slot_next = (tid < BN && j < sk.n_idx && j <= key_last) ? ((gptr<int64_t>)a.kv_indices)[kvs + j] : 0;
  };
  auto write_ptrs = [&](int kt) __attribute__((always_inline)) {
    if (tid < BN) {
      const int j = kt * BN + tid;
      gptr<T> kp = zrow;
      gptr<T> vp = zrow;
      if (j <= key_last) {
        if (j < sk.n_idx) {
          kp = kpool + slot_next * a.kp_ss + (int64_t)g * a.kp_sh;
          vp = vpool + slot_next * a.vp_ss + (int64_t)g * a.vp_sh;
        } else {
          const int64_t row = q0 + (j - P);
          kp = kext + row * a.ke_st + (int64_t)g * a.ke_sh;
          vp = vext + row * a.ve_st + (int64_t)g * a.ve_sh;
        }
      }
      kptr[kt & 1][tid] = kp;
      vptr[kt & 1][tid] = vp;
    }
  };

  // ---- global -> register staging of one tile
  u32x4 kreg[C::K_PER_THREAD];
  u32x4 vreg[C::V_PER_THREAD];
  auto load_tile = [&](int kt) __attribute__((always_inline)) {
    const int buf = kt & 1;
#pragma unroll
    for (int u = 0; u < C::K_PER_THREAD; ++u) {
      const int c = tid + u * NT;
      if (C::KC % NT == 0 || c < C::KC) {
        const int row = c / (LQ / VEC), col = (c % (LQ / VEC)) * VEC;
        kreg[u] = *(gptr<u32x4>)(kptr[buf][row] + col);
      }
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_THREAD; ++u) {
      const int c = tid + u * NT;
      if (C::VC % NT == 0 || c < C::VC) {
        const int row = c / (LV / VEC), col = (c % (LV / VEC)) * VEC;
        vreg[u] = *(gptr<u32x4>)(vptr[buf][row] + col);
      }
    }
  };
  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < C::K_PER_THREAD; ++u) {
      const int c = tid + u * NT;
      if (C::KC % NT == 0 || c < C::KC) {
        const int row = c / (LQ / VEC), col = (c % (LQ / VEC)) * VEC;
        if constexpr (F32) {
          float* dst = Ks + row * KROW + col;
          dst[0] = __uint_as_float(kreg[u][0]);
          dst[1] = __uint_as_float(kreg[u][1]);
          dst[2] = __uint_as_float(kreg[u][2]);
          dst[3] = __uint_as_float(kreg[u][3]);
        } else {
          *reinterpret_cast<u32x4*>(Ks + row * KROW + col) = kreg[u];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_THREAD; ++u) {
      const int c = tid + u * NT;
      if (C::VC % NT == 0 || c < C::VC) {
        const int row = c / (LV / VEC), col = (c % (LV / VEC)) * VEC;
        if constexpr (F32) {
          float* dst = Vs + row * VROW + col;
          dst[0] = __uint_as_float(vreg[u][0]);
          dst[1] = __uint_as_float(vreg[u][1]);
          dst[2] = __uint_as_float(vreg[u][2]);
          dst[3] = __uint_as_float(vreg[u][3]);
        } else {
          *reinterpret_cast<u32x4*>(Vs + row * VROW + col) = vreg[u];
        }
      }
    }
  };

  // prologue: pointer tables for the first two tiles, then the first tile's loads
  if (kt0 < kt1) {
    fetch_slot(kt0);
    write_ptrs(kt0);
    if (kt0 + 1 < kt1) {
      fetch_slot(kt0 + 1);
      write_ptrs(kt0 + 1);
    }
    __syncthreads();
    load_tile(kt0);
  }

  for (int kt = kt0; kt < kt1; ++kt) {
    __syncthreads();  // previous tile consumed; pointer table of kt+1 published
    store_tile();
    __syncthreads();
    if (kt + 1 < kt1) load_tile(kt + 1);  // in flight while this tile is computed
    if (kt + 2 < kt1) fetch_slot(kt + 2);

    const int j0 = kt * BN;
    if (wave_live && j0 <= lim_hi_w && j0 + BN - 1 >= lo_lo_w) {
      const bool need_mask = j0 + BN - 1 > lim_lo_w || j0 < lo_hi_w || !causal;

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

      // soft-cap (base-2 units), then mask the diagonal tiles, then the row max;
      // without a cap the max is taken on raw dot products and scaled after
      if constexpr (CAP) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const float e = fast_exp2(s[kb][rr] * (a.cap_in * 2.0f * kLog2e));
            s[kb][rr] = a.cap_out * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
          }
      }
      if (need_mask && causal) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int j = j0 + kb * 32 + 8 * (rr / 4) + 4 * hi + (rr % 4);
            s[kb][rr] = (j <= lim && j >= lo) ? s[kb][rr] : -INFINITY;
          }
      } else if (need_mask) {
        // custom mask: this row's bytes, key j at mrow[j] (addressed inside the
        // branch, so that calls without a mask hold no register for it)
        const uint8_t* mrow = a.custom_mask + a.mask_indptr[b] + (int64_t)tok * sk.n_keys;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int j = j0 + kb * 32 + 8 * (rr / 4) + 4 * hi + (rr % 4);
            s[kb][rr] = (j <= lim && j >= lo && mrow[j] != 0) ? s[kb][rr] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[kb][rr]);
      mx = pair_max(mx);
      if constexpr (!CAP) mx *= a.scale_log2;
      // raise the reference max only when some row outgrows it by the slack
      if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleSlack)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      }
      const float m_sub = m_ref == -INFINITY ? 0.0f : m_ref;

      // P and O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if constexpr (F32) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const float p = CAP ? fast_exp2(s[kb][rr] - m_sub) : fast_exp2(fmaf(s[kb][rr], a.scale_log2, -m_sub));
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
              const float x = s[kb][8 * half + e];
              const float p = CAP ? fast_exp2(x - m_sub) : fast_exp2(fmaf(x, a.scale_log2, -m_sub));
              pb[e] = (__bf16)p;
            }
            // the row sum adds the same rounded weights that multiply V, two per dot2
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), ones, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), ones, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), ones, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), ones, l_run, false);
            // keys kb*32 + 16*half + 4*hi + {0..3} and {8..11}: lane (in its 16-lane
            // group) j points at row key0 + j/4, columns cbase + 4*(j%4); it receives
            // the 4 keys of column cbase + j.
            const int key0 = kb * 32 + 16 * half + 4 * hi + ((lane & 15) >> 2);
            const int cofs = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const T* v0 = Vs + key0 * VROW + db * 32 + cofs;
              i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) i16x4*)(v0));
              i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) i16x4*)(v0 + 8 * VROW));
              bf16x8 va = __builtin_bit_cast(
                  bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc[db], 0, 0, 0);
            }
          }
        }
      }
    }
    if (kt + 2 < kt1) write_ptrs(kt + 2);  // its table slot was last read before this tile's barriers
  }

  // ---- epilogue
  const float l_tot = pair_sum(l_run);
  if (it.part < 0) {
    if (!valid) return;
    // a sink joins the denominator once, here or in the merge of split chunks
    const float inv = 1.0f / (a.sinks ? l_tot + fast_exp2(a.sinks[head] * kLog2e - m_ref) : l_tot);
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
    // (the merge reads only rows of the item's tokens: padding rows write nothing)
    if (!valid) return;
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
    if (hi == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(m_ref, l_tot);
  }
}

template <bool F32, int LQ, int LV, int BN, int MINB>
hipError_t launch_attn_t(const AttnArgs& a, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid), t(256);
  if (a.custom_mask || a.window > 0) {
    if (a.use_cap)
      hipLaunchKernelGGL((attn_kernel<F32, LQ, LV, BN, true, true, MINB>), g, t, 0, s, a);
    else
      hipLaunchKernelGGL((attn_kernel<F32, LQ, LV, BN, false, true, MINB>), g, t, 0, s, a);
  } else if (a.use_cap) {
    hipLaunchKernelGGL((attn_kernel<F32, LQ, LV, BN, true, false, MINB>), g, t, 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<F32, LQ, LV, BN, false, false, MINB>), g, t, 0, s, a);
  }
  return hipGetLastError();
}

template <bool F32, int LQ, int LV, int BN, int MINB>
int occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_kernel<F32, LQ, LV, BN, false, false, MINB>, 256, 0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

// The supported (dtype, lq, lv) variants: key-tile width and workgroups per CU.
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

hipError_t launch_split_merge(int dtype, int lv, int bm, const AttnArgs& a, hipStream_t s) {
  const dim3 g(512), t(256);  // a grid stride over (merge record, row block) tasks
  if (lv <= 0 || lv % 4 != 0) return hipErrorInvalidValue;
  if (dtype == 1) {
    if (lv <= 64) hipLaunchKernelGGL((split_merge_kernel<true, 64>), g, t, 0, s, a, bm, lv);
    else if (lv <= 128) hipLaunchKernelGGL((split_merge_kernel<true, 128>), g, t, 0, s, a, bm, lv);
    else return hipErrorInvalidValue;
  } else {
    if (lv <= 64) hipLaunchKernelGGL((split_merge_kernel<false, 64>), g, t, 0, s, a, bm, lv);
    else if (lv <= 128) hipLaunchKernelGGL((split_merge_kernel<false, 128>), g, t, 0, s, a, bm, lv);
    else if (lv <= 256) hipLaunchKernelGGL((split_merge_kernel<false, 256>), g, t, 0, s, a, bm, lv);
    else if (lv <= 512) hipLaunchKernelGGL((split_merge_kernel<false, 512>), g, t, 0, s, a, bm, lv);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

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

}  // namespace pkv
