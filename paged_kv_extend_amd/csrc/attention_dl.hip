// Extend-attention kernel for bf16 head dims 64, 128 and 256 on gfx950 with
// K/V tiles loaded straight from global memory into LDS.
//
// Same computation as attention.hip (page "extend_attention.py",
// _fwd_kernel_unified: scale, optional soft-cap, mask j <= P + i, online
// softmax with probabilities rounded to the value dtype; page
// "flashinfer_backend.py", forward_extend: prefix through kv_indices, new
// tokens through qo_indptr), with the same MFMA formulation: S^T = K Q^T and
// O^T = V^T P^T on 32x32x16 bf16 MFMA, one query row per lane.
//
// What differs from attention.hip is the tile movement:
//  * global_load_lds (16 bytes per lane) writes each K/V row chunk directly
//    into LDS: no staging registers, no LDS store instructions, and one barrier
//    per tile instead of two.  Two LDS stages: tile t+1 streams in while tile t
//    is computed.
//  * The load places lane L's 16 bytes at base + 16 L, so rows cannot be
//    padded; instead the 16-byte chunk index is XOR-swizzled per row (applied
//    when choosing each lane's global address, undone on reads): the
//    MFMA operand reads of K and the transposing reads of V stay free of bank
//    conflicts.
//  * Waits on the loads are explicit vmcnt counts before a bare s_barrier.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <class T>
using gptr = const __attribute__((address_space(1))) T*;
template <class T>
using lptr = __attribute__((address_space(3))) T*;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(0) lgkmcnt(0) (gfx9 encoding: vmcnt [3:0],[15:14]; expcnt [6:4]; lgkmcnt [11:8])
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0x7 << 4); }

template <int LQ, int LV, int BN>
struct DlCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;
  static constexpr int CK = LQ / 8;  // 16-byte chunks per row
  static constexpr int CV = LV / 8;
  // rows sharing one 256-byte window of the 64 LDS banks
  static constexpr int RPK = CK >= 16 ? 1 : 16 / CK;
  static constexpr int RPV = CV >= 16 ? 1 : 16 / CV;
  static constexpr int SWK = CK >= 16 ? 16 : CK;     // distinct K swizzles
  static constexpr int SWV = CV >= 16 ? 4 : CV / 4;  // distinct V swizzles (multiples of 4 chunks)
  static constexpr int K_BYTES = BN * LQ * 2;
  static constexpr int V_BYTES = BN * LV * 2;
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr int K_LOADS = K_BYTES / 1024 / NW;  // 1 KB load instructions per wave per tile
  static constexpr int V_LOADS = V_BYTES / 1024 / NW;
  static_assert(CK == 8 || CK == 16 || CK == 32, "lq");
  static_assert(CV == 8 || CV == 16 || CV == 32, "lv");
  static_assert(K_BYTES % (1024 * NW) == 0 && V_BYTES % (1024 * NW) == 0, "whole loads per wave");
  static_assert(BN % 32 == 0 && BN <= 64, "key tile");
};

// Physical 16-byte chunk of logical chunk c in row r.  K: the 32 rows read at
// one logical chunk by an MFMA operand load spread over all 16 bank groups.
// V: the 4 rows x 4 chunks of one transposing read spread over all 16 groups.
template <class C>
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ ((r / C::RPK) % C::SWK); }
template <class C>
__device__ __forceinline__ int swz_v(int r, int c) { return c ^ (4 * ((r / C::RPV) % C::SWV)); }

template <int LQ, int LV, int BN, bool CAP, int MINB>
__global__ __launch_bounds__(256, MINB) void attn_dl_kernel(AttnArgs a) {
  using C = DlCfg<LQ, LV, BN>;
  using T = uint16_t;
  constexpr int NT = C::NT, BM = C::BM;
  constexpr int NKB = BN / 32;
  constexpr int NQ = LQ / 16;
  constexpr int NDB = LV / 32;

  __shared__ __attribute__((aligned(1024))) char lds[2 * C::STAGE_BYTES];
  __shared__ gptr<T> kptr[2][BN];
  __shared__ gptr<T> vptr[2][BN];
  (void)NT;

  if ((int)blockIdx.x >= a.hdr->num_work) return;
  const WorkItem it = a.work[blockIdx.x];
  if (it.b < 0) return;  // empty placement slot
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int qi = lane & 31, hi = lane >> 5;
  const int G = a.group;
  const int b = it.b, g = it.g;
  const int q0 = a.qo_indptr[b], E = a.qo_indptr[b + 1] - q0;
  const int kvs = a.kv_indptr[b], P = a.kv_indptr[b + 1] - kvs;
  const int R = E * G;

  const int r = it.t * BM + wv * 32 + qi;
  const bool valid = r < R;
  const int lim = valid ? P + r / G : -1;  // last visible key of this lane's row
  const int rw0 = it.t * BM + wv * 32;
  const bool wave_live = rw0 < R;
  const int i_lo_w = wave_live ? rw0 / G : 0;
  const int i_hi_w = wave_live ? min(R - 1, rw0 + 31) / G : 0;
  const int key_last = P + min(R - 1, it.t * BM + BM - 1) / G;

  const gptr<T> kpool = (gptr<T>)a.k_pool;
  const gptr<T> vpool = (gptr<T>)a.v_pool;
  const gptr<T> kext = (gptr<T>)a.k_ext;
  const gptr<T> vext = (gptr<T>)a.v_ext;
  const gptr<T> zrow = (gptr<T>)a.zero_row;
  const int kt0 = it.kt_begin, kt1 = it.kt_end;

  // ---- Q^T operand (B) in registers, negated when the scale is negative
  bf16x8 qr[NQ];
  {
    const uint32_t flip = a.neg_q ? 0x80008000u : 0u;
    gptr<T> qrow = (gptr<T>)a.q + (int64_t)(q0 + (valid ? r / G : 0)) * a.q_st +
                   (int64_t)(g * G + (valid ? r % G : 0)) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
      const u32x4 v = valid ? *(gptr<u32x4>)(qrow + ks * 16 + hi * 8) : u32x4{0u, 0u, 0u, 0u};
      qr[ks] = __builtin_bit_cast(bf16x8, v ^ flip);
    }
  }

  // ---- row pointer tables (two slots); lane j < BN of the owning wave owns key kt*BN + j
  int64_t slot_next = 0;
  auto fetch_slot = [&](int kt) __attribute__((always_inline)) {
    const int j = kt * BN + lane;
    slot_next = (lane < BN && j < P && j <= key_last) ? ((gptr<int64_t>)a.kv_indices)[kvs + j] : 0;
  };
  auto write_ptrs = [&](int kt) __attribute__((always_inline)) {
    if (lane < BN) {
      const int j = kt * BN + lane;
      gptr<T> kp = zrow;
      gptr<T> vp = zrow;
      if (j <= key_last) {
        if (j < P) {
          kp = kpool + slot_next * a.kp_ss + (int64_t)g * a.kp_sh;
          vp = vpool + slot_next * a.vp_ss + (int64_t)g * a.vp_sh;
        } else {
          const int64_t row = q0 + (j - P);
          kp = kext + row * a.ke_st + (int64_t)g * a.ke_sh;
          vp = vext + row * a.ve_st + (int64_t)g * a.ve_sh;
        }
      }
      kptr[kt & 1][lane] = kp;
      vptr[kt & 1][lane] = vp;
    }
  };

  // ---- direct loads of tile kt into stage kt & 1: wave w covers bytes
  //      [(i * NW + w) * 1024, +1024) of the K and V regions
  auto issue_tile = [&](int kt) __attribute__((always_inline)) {
    char* stage = lds + (kt & 1) * C::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int base = (i * C::NW + wv) * 1024;
      const int off = base + lane * 16;
      const int row = off / (LQ * 2), p = (off % (LQ * 2)) / 16;
      __builtin_amdgcn_global_load_lds((gptr<void>)(kptr[kt & 1][row] + swz_k<C>(row, p) * 8),
                                       (lptr<void>)(stage + base), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
      const int base = (i * C::NW + wv) * 1024;
      const int off = base + lane * 16;
      const int row = off / (LV * 2), p = (off % (LV * 2)) / 16;
      __builtin_amdgcn_global_load_lds((gptr<void>)(vptr[kt & 1][row] + swz_v<C>(row, p) * 8),
                                       (lptr<void>)(stage + C::K_BYTES + base), 16, 0, 0);
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_ref = -INFINITY;  // reference max of the exponentials, base-2 units
  float l_run = 0.0f;       // this lane's share of the running sum

  if (kt0 < kt1) {
    if (wv < 2 && kt0 + wv < kt1) {  // tables of the first two tiles, one wave each
      fetch_slot(kt0 + wv);
      write_ptrs(kt0 + wv);
    }
    __syncthreads();
    issue_tile(kt0);
  }

  for (int kt = kt0; kt < kt1; ++kt) {
    // only tile kt's loads are outstanding here (the index load of the wave
    // that builds tables was waited for when its table was written)
    wait_all_mem();
    __builtin_amdgcn_s_barrier();  // tile kt visible; stage and table of kt+1 free/visible
    if (wv == 0 && kt + 2 < kt1) fetch_slot(kt + 2);  // before the tile loads: waiting for it never waits for them
    if (kt + 1 < kt1) issue_tile(kt + 1);

    const int j0 = kt * BN;
    if (wave_live && j0 <= P + i_hi_w) {
      const bool need_mask = j0 + BN - 1 > P + i_lo_w;
      const char* Ks = lds + (kt & 1) * C::STAGE_BYTES;
      const char* Vs = Ks + C::K_BYTES;

      // S^T = K Q^T
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int row = kb * 32 + qi;
          const bf16x8 kv = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(Ks + row * LQ * 2 + swz_k<C>(row, 2 * ks + hi) * 16));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qr[ks], s[kb], 0, 0, 0);
        }
      }

      // soft-cap (base-2 units), mask of the diagonal tiles, row max
      if constexpr (CAP) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const float e = fast_exp2(s[kb][rr] * (a.cap_in * 2.0f * kLog2e));
            s[kb][rr] = a.cap_out * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
          }
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int j = j0 + kb * 32 + 8 * (rr / 4) + 4 * hi + (rr % 4);
            s[kb][rr] = j <= lim ? s[kb][rr] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[kb][rr]);
      mx = pair_max(mx);
      if constexpr (!CAP) mx *= a.scale_log2;
      if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleSlack)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      }
      const float m_sub = m_ref == -INFINITY ? 0.0f : m_ref;

      // P (bf16, summed with dot2) and O^T += V^T P^T
      const int key0 = 4 * hi + ((lane & 15) >> 2);
      const int cofs = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = s[kb][8 * half + e];
            const float p = CAP ? fast_exp2(x - m_sub) : fast_exp2(fmaf(x, a.scale_log2, -m_sub));
            pb[e] = (__bf16)p;
          }
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), ones, l_run, false);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), ones, l_run, false);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), ones, l_run, false);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), ones, l_run, false);
          const int r0 = kb * 32 + 16 * half + key0, r1 = r0 + 8;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int col = db * 32 + cofs;
            const char* a0 = Vs + r0 * LV * 2 + swz_v<C>(r0, col / 8) * 16 + (col % 8) * 2;
            const char* a1 = Vs + r1 * LV * 2 + swz_v<C>(r1, col / 8) * 16 + (col % 8) * 2;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr<i16x4>)(a0));
            const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr<i16x4>)(a1));
            const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc[db], 0, 0, 0);
          }
        }
      }
    }
    // table of kt+2 into the slot of kt (last read when tile kt was issued)
    if (wv == 0 && kt + 2 < kt1) write_ptrs(kt + 2);
  }

  // ---- epilogue
  const float l_tot = pair_sum(l_run);
  if (it.part < 0) {
    if (!valid) return;
    const float inv = 1.0f / l_tot;
    T* orow = reinterpret_cast<T*>(a.o) + (int64_t)(q0 + r / G) * a.o_st + (int64_t)(g * G + r % G) * a.o_sh;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hi;
        bf16x4 ov;
        ov[0] = (__bf16)(acc[db][4 * g4] * inv);
        ov[1] = (__bf16)(acc[db][4 * g4 + 1] * inv);
        ov[2] = (__bf16)(acc[db][4 * g4 + 2] * inv);
        ov[3] = (__bf16)(acc[db][4 * g4 + 3] * inv);
        *reinterpret_cast<bf16x4*>(orow + d) = ov;
      }
    }
  } else {
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

template <int LQ, int LV, int BN, int MINB>
hipError_t launch_dl_t(const AttnArgs& a, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (a.use_cap)
    hipLaunchKernelGGL((attn_dl_kernel<LQ, LV, BN, true, MINB>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_dl_kernel<LQ, LV, BN, false, MINB>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int LQ, int LV, int BN, int MINB>
int dl_occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&attn_dl_kernel<LQ, LV, BN, false, MINB>), 256, 0) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

// bf16 (lq, lv) pairs served here: key-tile width and workgroups per CU
#define PKV_DL_VARIANTS(X) \
  X(64, 64, 64, 2)         \
  X(128, 128, 64, 2)       \
  X(256, 256, 32, 1)

}  // namespace

bool dl_tiling(int dtype, int lq, int lv, Tiling* t) {
  if (dtype != 0) return false;
#define PKV_DT(Q, V, N, M)           \
  if (lq == Q && lv == V) {          \
    t->bm = DlCfg<Q, V, N>::BM;      \
    t->bn = N;                       \
    t->threads = 256;                \
    return true;                     \
  }
  PKV_DL_VARIANTS(PKV_DT)
#undef PKV_DT
  return false;
}

hipError_t launch_dl(int lq, int lv, const AttnArgs& a, int64_t grid, hipStream_t s) {
#define PKV_DLL(Q, V, N, M) \
  if (lq == Q && lv == V) return launch_dl_t<Q, V, N, M>(a, grid, s);
  PKV_DL_VARIANTS(PKV_DLL)
#undef PKV_DLL
  return hipErrorInvalidValue;
}

int dl_blocks_per_cu(int lq, int lv) {
#define PKV_DLO(Q, V, N, M) \
  if (lq == Q && lv == V) return dl_occupancy_t<Q, V, N, M>();
  PKV_DL_VARIANTS(PKV_DLO)
#undef PKV_DLO
  return 1;
}

}  // namespace pkv
