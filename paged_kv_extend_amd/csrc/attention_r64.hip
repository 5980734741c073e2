// Extend-attention kernel for bf16 head dim 128 on gfx950: 64 query rows per
// wave, one wave per SIMD, a skewed software pipeline.
//
// Same computation as attention.hip (page "extend_attention.py",
// _fwd_kernel_unified: scale, optional soft-cap, mask j <= P + i, online
// softmax with probabilities rounded to the value dtype; page
// "flashinfer_backend.py", forward_extend: prefix through kv_indices, new
// tokens through qo_indptr) and the same MFMA formulation (S^T = K Q^T and
// O^T = V^T P^T on 32x32x16 bf16 MFMA, one query row per lane).  What differs:
//  * A wave owns 64 packed query rows (two 32-row blocks), so every K or V
//    operand read from LDS feeds two MFMAs.  With 32 rows per wave the LDS
//    operand traffic (1 KB per MFMA) exceeds what LDS delivers at the MFMA
//    rate; with 64 it is half that.
//  * One wave per SIMD (two 2-wave workgroups per CU) gives each wave the
//    512-entry register file for two Q^T blocks, two O^T blocks and two tiles
//    of S.
//  * The loop is skewed so that one wave keeps the matrix core busy during
//    its own softmax: iteration t issues S(t+1) = K(t+1) Q^T, then takes the
//    softmax of S(t) (computed one iteration earlier) and O += P(t) V(t).
//    K and V have separate double-buffered LDS stages; K(t+2) and V(t+1) are
//    issued at the top of iteration t, a whole iteration before their use.
//  * Tiles move straight from global memory into LDS (global_load_lds,
//    16 bytes per lane) with the XOR chunk swizzles that keep the MFMA operand
//    reads and the transposing V reads free of bank conflicts.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <int D, int BN>
struct R64Cfg {
  static constexpr int NW = 2;  // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int RS = 2;  // 32-row blocks per wave
  static constexpr int BM = NW * RS * 32;
  static constexpr int CH = D / 8;  // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int LOADS = TILE_BYTES / 1024 / NW;  // 1 KB loads per wave per K or V tile
  static_assert(CH == 16, "swizzles below are for 256-byte rows");
  static_assert(TILE_BYTES % (1024 * NW) == 0, "whole loads per wave");
  static_assert(BN % 32 == 0 && BN <= 64, "key tile");
};

// Physical 16-byte chunk of logical chunk c in row r (256-byte rows).  K: the
// 32 rows that one MFMA operand read touches at one logical chunk spread over
// all 16 bank groups.  V: the 4 rows x 4 chunks of one transposing read do.
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_v(int r, int c) { return c ^ (4 * (r & 3)); }

template <int D, int BN, bool CAP>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_r64_kernel(AttnArgs a) {
  using C = R64Cfg<D, BN>;
  using T = uint16_t;
  constexpr int BM = C::BM, RS = C::RS;
  constexpr int NKB = BN / 32;
  constexpr int NQ = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TB = C::TILE_BYTES;

  // K stages 0, 1 then V stages 0, 1
  __shared__ __attribute__((aligned(1024))) char lds[4 * TB];
  __shared__ gptr<T> kptr[4][BN];
  __shared__ gptr<T> vptr[4][BN];

  if ((int)blockIdx.x >= a.hdr->num_work) return;
  const WorkItem it = a.work[blockIdx.x];
  if (it.b < 0) return;  // empty placement slot
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
  const int qi = lane & 31, hi = lane >> 5;
  const int G = a.group;
  const int b = it.b, g = it.g;
  const SeqKeys sk = seq_keys(a.qo_indptr, a.kv_indptr, a.prefix_lens, b);
  const int q0 = sk.q0, E = sk.E, kvs = sk.kvs, P = sk.P;
  const int R = E * G;

  const int rw0 = it.t * BM + wv * 64;  // first row of this wave
  int lim[RS];
  bool valid[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int r = rw0 + rs * 32 + qi;
    valid[rs] = r < R;
    lim[rs] = valid[rs] ? min(P + r / G, sk.n_keys - 1) : -1;  // last visible key of this lane's row
  }
  const bool wave_live = rw0 < R;
  const int lim_lo_w = min(P + (wave_live ? rw0 / G : 0), sk.n_keys - 1);
  const int lim_hi_w = min(P + (wave_live ? min(R - 1, rw0 + 63) / G : 0), sk.n_keys - 1);
  const int key_last = min(P + min(R - 1, it.t * BM + BM - 1) / G, sk.n_keys - 1);

  const gptr<T> kpool = (gptr<T>)a.k_pool;
  const gptr<T> vpool = (gptr<T>)a.v_pool;
  const gptr<T> kext = (gptr<T>)a.k_ext;
  const gptr<T> vext = (gptr<T>)a.v_ext;
  const gptr<T> zrow = (gptr<T>)a.zero_row;
  const int kt0 = it.kt_begin, kt1 = it.kt_end;

  // ---- Q^T operands (B) in registers, negated when the scale is negative
  bf16x8 qr[RS][NQ];
  {
    const uint32_t flip = a.neg_q ? 0x80008000u : 0u;
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      const int r = rw0 + rs * 32 + qi;
      gptr<T> qrow = (gptr<T>)a.q + (int64_t)(q0 + (valid[rs] ? r / G : 0)) * a.q_st +
                     (int64_t)(g * G + (valid[rs] ? r % G : 0)) * a.q_sh;
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) {
        const u32x4 v = valid[rs] ? *(gptr<u32x4>)(qrow + ks * 16 + hi * 8) : u32x4{0u, 0u, 0u, 0u};
        qr[rs][ks] = __builtin_bit_cast(bf16x8, v ^ flip);
      }
    }
  }

  // ---- row pointer tables, 4 slots; lane j < BN of the building wave owns key kt*BN + j
  int64_t slot_next = 0;
  auto fetch_slot = [&](int kt) __attribute__((always_inline)) {
    const int j = kt * BN + lane;
    slot_next = (lane < BN && j < sk.n_idx && j <= key_last) ? ((gptr<int64_t>)a.kv_indices)[kvs + j] : 0;
  };
  auto write_ptrs = [&](int kt) __attribute__((always_inline)) {
    if (lane < BN) {
      const int j = kt * BN + lane;
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
      kptr[kt & 3][lane] = kp;
      vptr[kt & 3][lane] = vp;
    }
  };

  // ---- direct loads: wave w covers bytes [(i * NW + w) * 1024, +1024) of a
  //      tile.  All row pointers are read before the first load is issued
  //      (each load is a compiler memory barrier).
  auto issue_k = [&](int kt) __attribute__((always_inline)) {
    const uint32_t st = lds_addr(lds + (kt & 1) * TB);
    gptr<T> src[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int off = (i * C::NW + wv) * 1024 + lane * 16;
      const int row = off / (D * 2), p = (off % (D * 2)) / 16;
      src[i] = kptr[kt & 3][row] + swz_k(row, p) * 8;
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) load_lds_16((gptr<void>)src[i], st + (i * C::NW + wv) * 1024);
  };
  auto issue_v = [&](int kt) __attribute__((always_inline)) {
    const uint32_t st = lds_addr(lds + (2 + (kt & 1)) * TB);
    gptr<T> src[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int off = (i * C::NW + wv) * 1024 + lane * 16;
      const int row = off / (D * 2), p = (off % (D * 2)) / 16;
      src[i] = vptr[kt & 3][row] + swz_v(row, p) * 8;
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) load_lds_16((gptr<void>)src[i], st + (i * C::NW + wv) * 1024);
  };

  auto active = [&](int kt) __attribute__((always_inline)) { return wave_live && kt * BN <= lim_hi_w; };
  auto needs_mask = [&](int kt) __attribute__((always_inline)) { return kt * BN + BN - 1 > lim_lo_w; };

  typedef f32x16 STile[RS][NKB];  // S^T of one key tile, both row blocks
  typedef bf16x8 PTile[NKB][2][RS];  // probabilities in B-operand layout

  // K operands of tile kt, all requested together
  auto read_k = [&](int kt, bf16x8 (&kv)[NQ][NKB]) __attribute__((always_inline)) {
    const char* Ks = lds + (kt & 1) * TB;
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = kb * 32 + qi;
        kv[ks][kb] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Ks + row * D * 2 + swz_k(row, 2 * ks + hi) * 16));
      }
  };
  // S^T = K Q^T
  auto qk_mfma = [&](const bf16x8 (&kv)[NQ][NKB], STile& s) __attribute__((always_inline)) {
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[rs][kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
          s[rs][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv[ks][kb], qr[rs][ks], s[rs][kb], 0, 0, 0);
  };
  // soft-cap, in base-2 units: cap * tanh(s * scale / cap) * log2(e)
  auto cap_tile = [&](STile& s) __attribute__((always_inline)) {
    if constexpr (CAP) {
#pragma unroll
      for (int rs = 0; rs < RS; ++rs)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const float e = fast_exp2(s[rs][kb][rr] * (a.cap_in * 2.0f * kLog2e));
            s[rs][kb][rr] = a.cap_out * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
          }
    }
  };
  // keys past a row's last visible key to -inf (tiles crossing the diagonal)
  auto mask_tile = [&](int kt, STile& s) __attribute__((always_inline)) {
    const int j0 = kt * BN;
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int j = j0 + kb * 32 + 8 * (rr / 4) + 4 * hi + (rr % 4);
          s[rs][kb][rr] = j <= lim[rs] ? s[rs][kb][rr] : -INFINITY;
        }
  };
  // row max over the tile (both lanes of a row)
  auto row_max = [&](const STile& s, float (&mx)[RS]) __attribute__((always_inline)) {
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) m = fmaxf(m, s[rs][kb][rr]);
      mx[rs] = pair_max(m);
    }
  };

  f32x16 acc[RS][NDB];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[rs][db] = f32x16{};
  float m_ref[RS], l_run[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    m_ref[rs] = -INFINITY;  // reference max of the exponentials, base-2 units
    l_run[rs] = 0.0f;       // this lane's share of the running sum
  }

  // raise the reference max of a row block where the tile's row max exceeds
  // it by more than the slack (rescaling O and the running sum); returns the
  // value subtracted in the exponent
  auto rescale = [&](const float (&mx)[RS], float (&m_sub)[RS]) __attribute__((always_inline)) {
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      const float m = CAP ? mx[rs] : mx[rs] * a.scale_log2;
      if (__builtin_amdgcn_ballot_w64(m > m_ref[rs] + kRescaleSlack)) {
        const float m_new = fmaxf(m_ref[rs], m);
        const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_ref[rs] - m_new);
        m_ref[rs] = m_new;
        l_run[rs] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[rs][db] *= alpha;
      }
      m_sub[rs] = m_ref[rs] == -INFINITY ? 0.0f : m_ref[rs];
    }
  };
  // probabilities rounded to bf16, and their sum (bf16 dot2 with ones)
  auto probs = [&](const STile& s, const float (&m_sub)[RS], PTile& pb) __attribute__((always_inline)) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
          bf16x8 q;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = s[rs][kb][8 * hf + e];
            const float p = CAP ? fast_exp2(x - m_sub[rs]) : fast_exp2(fmaf(x, a.scale_log2, -m_sub[rs]));
            q[e] = (__bf16)p;
          }
          l_run[rs] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 0, 1), ones, l_run[rs], false);
          l_run[rs] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 2, 3), ones, l_run[rs], false);
          l_run[rs] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 4, 5), ones, l_run[rs], false);
          l_run[rs] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 6, 7), ones, l_run[rs], false);
          pb[kb][hf][rs] = q;
        }
  };
  // V^T operands of tile kt (transposing LDS reads, 4 keys per lane)
  const int key0 = 4 * hi + ((lane & 15) >> 2);
  const int cofs = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto read_v = [&](int kt, bf16x8 (&va)[NKB][2][NDB]) __attribute__((always_inline)) {
    const char* Vs = lds + (2 + (kt & 1)) * TB;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int r0 = kb * 32 + 16 * hf + key0, r1 = r0 + 8;
          const int col = db * 32 + cofs;
          const char* a0 = Vs + r0 * D * 2 + swz_v(r0, col / 8) * 16 + (col % 8) * 2;
          const char* a1 = Vs + r1 * D * 2 + swz_v(r1, col / 8) * 16 + (col % 8) * 2;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr<i16x4>)(a0));
          const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr<i16x4>)(a1));
          va[kb][hf][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        }
  };
  // O^T += V^T P^T
  auto pv_mfma = [&](const bf16x8 (&va)[NKB][2][NDB], const PTile& pb) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int rs = 0; rs < RS; ++rs)
            acc[rs][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kb][hf][db], pb[kb][hf][rs], acc[rs][db], 0, 0, 0);
  };

  // One iteration: tile kt's softmax and P V, with tile kt+1's S = K Q^T
  // issued alongside.  On entry sc holds S(kt) (soft-capped) and mc its
  // unmasked row max; on exit sn and mn hold the same for kt+1.
  constexpr int kQkMfma = NQ * NKB * RS, kPvMfma = NKB * 2 * NDB * RS;
  auto step = [&](int kt, STile& sc, STile& sn, float (&mc)[RS], float (&mn)[RS]) __attribute__((always_inline)) {
    // outstanding: V(kt), K(kt+1).  After the barrier both are visible, K
    // stage kt & 1 (read by the S(kt) products) and V stage (kt+1) & 1 (read
    // by the P(kt-1) V products) are free, and so is table slot (kt+3) & 3.
    wait_all_mem();
    barrier_fence();
    if (wv == 0 && kt + 3 < kt1) fetch_slot(kt + 3);
    if (kt + 2 < kt1) issue_k(kt + 2);
    if (kt + 1 < kt1) issue_v(kt + 1);
    // Tiles a wave computes are a prefix of [kt0, kt1) (causal), so when
    // tile kt is active the products for kt+1 are made even when kt+1 is not:
    // they then read a stale but complete K stage and are never used.  One
    // code path keeps the register assignment the same on every trip.
    if (active(kt)) {
      float m_sub[RS];
      if (needs_mask(kt)) {
        mask_tile(kt, sc);
        row_max(sc, mc);
      }
      rescale(mc, m_sub);
      // Block A: the products of S(kt+1) with the probabilities of S(kt).
      // Unit u issues one MFMA and then two probabilities (FMA, exp, bf16
      // pack, dot2 into the row sum), which run on the VALU while the matrix
      // core works; sched_barrier keeps the order as written.
      bf16x8 kv[NQ][NKB];
      PTile pb;
      read_k(kt + 1, kv);
#pragma unroll
      for (int rs = 0; rs < RS; ++rs)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sn[rs][kb] = f32x16{};
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      static_assert(kQkMfma * 2 == NKB * 2 * RS * 8, "two probabilities per product");
#pragma unroll
      for (int u = 0; u < kQkMfma; ++u) {
        {
          const int ks = u / (NKB * RS), kb = (u / RS) % NKB, rs = u % RS;
          sn[rs][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv[ks][kb], qr[rs][ks], sn[rs][kb], 0, 0, 0);
        }
        {
          const int g = u / 4, e = 2 * (u % 4);  // probabilities e, e+1 of group g = (kb, hf, rs)
          const int kb = g / (2 * RS), hf = (g / RS) % 2, rs = g % RS;
          const float x0 = sc[rs][kb][8 * hf + e], x1 = sc[rs][kb][8 * hf + e + 1];
          const float p0 = CAP ? fast_exp2(x0 - m_sub[rs]) : fast_exp2(fmaf(x0, a.scale_log2, -m_sub[rs]));
          const float p1 = CAP ? fast_exp2(x1 - m_sub[rs]) : fast_exp2(fmaf(x1, a.scale_log2, -m_sub[rs]));
          const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
          l_run[rs] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run[rs], false);
          pb[kb][hf][rs][e] = pp[0];
          pb[kb][hf][rs][e + 1] = pp[1];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Block B: P(kt) V(kt) with the soft-cap and row max of S(kt+1).
      bf16x8 va[NKB][2][NDB];
      read_v(kt, va);
      float mrun[RS];
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) mrun[rs] = -INFINITY;
      constexpr int kVals = RS * NKB * 16;  // S values of a lane, capped and max-reduced
      constexpr int kPer = (kVals + kPvMfma - 1) / kPvMfma;
#pragma unroll
      for (int u = 0; u < kPvMfma; ++u) {
        {
          const int kb = u / (2 * NDB * RS), hf = (u / (NDB * RS)) % 2, db = (u / RS) % NDB, rs = u % RS;
          acc[rs][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kb][hf][db], pb[kb][hf][rs], acc[rs][db], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int v = u * kPer + k;
          if (v < kVals) {
            const int rs = v / (NKB * 16), kb = (v / 16) % NKB, rr = v % 16;
            float x = sn[rs][kb][rr];
            if constexpr (CAP) {
              const float e = fast_exp2(x * (a.cap_in * 2.0f * kLog2e));
              x = a.cap_out * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
              sn[rs][kb][rr] = x;
            }
            mrun[rs] = fmaxf(mrun[rs], x);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) mn[rs] = pair_max(mrun[rs]);
    }
    if (wv == 0 && kt + 3 < kt1) write_ptrs(kt + 3);
  };

  STile s_a, s_b;
  float m_a[RS], m_b[RS];
  if (kt0 < kt1) {
    // tables of the first three tiles
    if (wv == 0) {
      fetch_slot(kt0);
      write_ptrs(kt0);
      if (kt0 + 2 < kt1) {
        fetch_slot(kt0 + 2);
        write_ptrs(kt0 + 2);
      }
    } else if (wv == 1 && kt0 + 1 < kt1) {
      fetch_slot(kt0 + 1);
      write_ptrs(kt0 + 1);
    }
    __syncthreads();
    issue_k(kt0);
    issue_v(kt0);
    if (kt0 + 1 < kt1) {
      issue_k(kt0 + 1);
      wait_vm<2 * C::LOADS>();  // K(kt0) landed; V(kt0), K(kt0+1) may still fly
    } else {
      wait_vm<C::LOADS>();
    }
    barrier_fence();
    if (active(kt0)) {
      bf16x8 kv[NQ][NKB];
      read_k(kt0, kv);
      qk_mfma(kv, s_a);
      cap_tile(s_a);
      row_max(s_a, m_a);
    }
  }
  // two tiles per trip so that the S tiles swap roles without copies
  int kt = kt0;
  for (; kt + 1 < kt1; kt += 2) {
    step(kt, s_a, s_b, m_a, m_b);
    step(kt + 1, s_b, s_a, m_b, m_a);
  }
  if (kt < kt1) step(kt, s_a, s_b, m_a, m_b);

  // ---- epilogue
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const float l_tot = pair_sum(l_run[rs]);
    const int r = rw0 + rs * 32 + qi;
    if (it.part < 0) {
      if (valid[rs]) {
        const float inv = 1.0f / l_tot;
        T* orow =
            reinterpret_cast<T*>(a.o) + (int64_t)(q0 + r / G) * a.o_st + (int64_t)(g * G + r % G) * a.o_sh;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d = db * 32 + 8 * g4 + 4 * hi;
            bf16x4 ov;
            ov[0] = (__bf16)(acc[rs][db][4 * g4] * inv);
            ov[1] = (__bf16)(acc[rs][db][4 * g4 + 1] * inv);
            ov[2] = (__bf16)(acc[rs][db][4 * g4 + 2] * inv);
            ov[3] = (__bf16)(acc[rs][db][4 * g4 + 3] * inv);
            *reinterpret_cast<bf16x4*>(orow + d) = ov;
          }
        }
      }
    } else {
      const int64_t prow = (int64_t)it.part * BM + (r - it.t * BM);
      float* pa = a.part_acc + prow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hi;
          *reinterpret_cast<float4*>(pa + d) = make_float4(acc[rs][db][4 * g4], acc[rs][db][4 * g4 + 1],
                                                           acc[rs][db][4 * g4 + 2], acc[rs][db][4 * g4 + 3]);
        }
      }
      if (hi == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(m_ref[rs], l_tot);
    }
  }
}

template <int D, int BN>
hipError_t launch_r64_t(const AttnArgs& a, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (a.use_cap)
    hipLaunchKernelGGL((attn_r64_kernel<D, BN, true>), dim3((unsigned)grid), dim3(R64Cfg<D, BN>::NT), 0, s, a);
  else
    hipLaunchKernelGGL((attn_r64_kernel<D, BN, false>), dim3((unsigned)grid), dim3(R64Cfg<D, BN>::NT), 0, s, a);
  return hipGetLastError();
}

template <int D, int BN>
int r64_occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&attn_r64_kernel<D, BN, false>), R64Cfg<D, BN>::NT, 0) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

// bf16 variants served here: (head dim for both Q/K and V, key tile)
#define PKV_R64_VARIANTS(X) X(128, 32)

}  // namespace

bool r64_tiling(int dtype, int lq, int lv, Tiling* t) {
  if (dtype != 0 || lq != lv) return false;
#define PKV_RT(D, N)                \
  if (lq == D) {                    \
    t->bm = R64Cfg<D, N>::BM;       \
    t->bn = N;                      \
    t->threads = R64Cfg<D, N>::NT;  \
    return true;                    \
  }
  PKV_R64_VARIANTS(PKV_RT)
#undef PKV_RT
  return false;
}

hipError_t launch_r64(int lq, const AttnArgs& a, int64_t grid, hipStream_t s) {
#define PKV_RL(D, N) \
  if (lq == D) return launch_r64_t<D, N>(a, grid, s);
  PKV_R64_VARIANTS(PKV_RL)
#undef PKV_RL
  return hipErrorInvalidValue;
}

int r64_blocks_per_cu(int lq) {
#define PKV_RO(D, N) \
  if (lq == D) return r64_occupancy_t<D, N>();
  PKV_R64_VARIANTS(PKV_RO)
#undef PKV_RO
  return 1;
}

}  // namespace pkv
