// Decode attention for bf16 on gfx950: one query token per request over the
// request's pool keys, the keys split into chunks that run in parallel and a
// log-sum-exp merge of the chunks.
//
// Page "flashinfer_backend.py": forward_decode attends each request's single
// new token to every key the decode index updater lists for it (the new
// token's own K/V already stored in the pool); the sliding-window updater
// keeps only the last window + 1 keys.  Scale, soft-cap and sinks as in page
// "extend_attention.py", _fwd_kernel_unified.  The merge of chunk states is
// the merge_state of page "flashinfer_backend.py", forward_extend.
//
// Decode moves every key's K/V row once and does little arithmetic per byte
// (2 (lq + lv) G flops per key and KV head), so the kernel is built to keep
// HBM busy:
//  * A plan launch (one workgroup) writes each request's first visible key in
//    the concatenation of all requests' visible keys.  The attention launch
//    cuts that concatenation into equal chunks of keys: grid (KV head x head
//    block, chunk), sized on the host to about one workgroup per CU whatever
//    the length mix; a request longer than a chunk spreads over several.
//  * Inside a workgroup each of the (usually four) waves streams its own contiguous
//    share of the chunk's keys, 16 keys per tile, through a ring of LDS stages
//    filled by global-to-LDS loads (16 bytes per lane, whole rows per group of
//    lanes).  A stage is refilled as soon as the wave is done with it,
//    before the wave waits for its next tile, so that every stage is in
//    flight during that wait.  The slots of later tiles come into LDS the
//    same way, far enough ahead that every wait in the loop is a fixed vmcnt,
//    and no wave waits for another until the chunk is done.
//  * The G query heads of a KV head (padded to 16) form the N side of 16x16
//    MFMAs: S^T = K Q^T on 16x16x32 bf16 with K read from LDS, O^T = V^T P^T
//    on 16x16x16 bf16 with V^T read by the transposing LDS read; the
//    probabilities already sit in the B-operand layout.  Each lane holds four
//    keys of one head, so a head's max and sum take two lane exchanges.
//  * The four waves' states are merged through LDS; a request wholly inside
//    the chunk is normalised and written out, otherwise the chunk writes its
//    unnormalised state, and a merge launch (a workgroup per request, head
//    block and 64-column slice, many in parallel) combines a request's chunks
//    in chunk order (deterministic) and writes zeros for requests without
//    keys.  Keeping the merge out of the attention launch spares
//    its workgroups the fences and counters, and a long request's many
//    partial states are read by a whole workgroup instead of one straggler.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kTile = 16;  // keys per wave per stage: the M side of the 16x16 MFMAs

template <int LQ, int LV, bool VK, int NW, int NS>
struct DecCfg {
  static constexpr int CK = LQ / 8;  // 16-byte chunks per K row
  static constexpr int CV = LV / 8;
  static constexpr int K_LOADS = kTile * CK / 64;  // 1 KB global-to-LDS loads per tile
  static constexpr int V_LOADS = VK ? 0 : kTile * CV / 64;
  static constexpr int L = K_LOADS + V_LOADS + 1;  // loads per trip: the tile's rows and one slot table
  static constexpr int K_BYTES = kTile * LQ * 2;
  static constexpr int STAGE = K_BYTES + (VK ? 0 : kTile * LV * 2);
  static constexpr int NSI = 2 * NS;  // slot tables in the ring
  static constexpr int SLOT_BYTES = 256;  // one table: 16 int64 slots, written twice (all 64 lanes load)
  static constexpr int WAVE_BYTES = NS * STAGE + NSI * SLOT_BYTES;
  // the waves' states for their merge: (m, l) of 16 rows, then the 16 rows'
  // accumulators at a pitch of LV + 4 floats (16 bytes of padding put the 16
  // rows one 16-byte write touches on distinct LDS banks)
  static constexpr int MP = LV + 4;
  static constexpr int MERGE_BYTES = NW * 16 * (2 + MP) * 4;
  static constexpr int LDS = NW * WAVE_BYTES > MERGE_BYTES ? NW * WAVE_BYTES : MERGE_BYTES;
  static constexpr int NT = NW * 64;
  // loads that may stay in flight in trip t (which issues tile t + NS - 1
  // before it waits for tile t): once the slot table of tile t + NS - 1 has
  // landed, the NS - 1 trips issued after it; once tile t has landed, the
  // slot table requested right after it and NS - 1 whole trips
  static constexpr int W_SLOTS = (NS - 1) * L;
  static constexpr int W_TILE = 1 + (NS - 1) * L;
  static_assert(LQ % 32 == 0 && LV % 16 == 0, "head dims");
  static_assert(VK ? LV <= LQ : CV % 4 == 0, "lv");
  static_assert(NS >= 2 && W_TILE < 64, "pipeline depth");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// XOR applied to the 16-byte chunk index of LDS row r, chosen per row pitch so
// that the 16 rows one operand read touches spread over the LDS banks; an
// involution inside an aligned group of chunks that divides the row.
template <int C>
__device__ __forceinline__ unsigned swz_k(unsigned r) {
  if constexpr (C % 16 == 0) {
    return r % 16u;
  } else if constexpr (C % 8 == 0) {
    return (r / 2u) % 8u;  // pitch = 8 chunks mod 16: rows pair up in a bank window
  } else {
    return (r / 4u) % 4u;  // pitch = 4 or 12 chunks mod 16
  }
}
// V rows: even values keep the 32-byte column pair of one transposing read together
template <int C>
__device__ __forceinline__ unsigned swz_v(unsigned r) {
  if constexpr (C % 16 == 0) {
    return 2u * (r % 8u);
  } else {
    return 2u * ((r / 2u) % 4u);  // 8 chunks per row
  }
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }

__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int carry = 0;
  for (int base = 0; base < a.bs; base += 1024) {
    const int b = base + tid;
    int v = 0;
    if (b < a.bs) {
      const int n = a.kv_indptr[b + 1] - a.kv_indptr[b];
      v = (a.window > 0 && n - 1 > a.window) ? a.window + 1 : n;  // (no overflow at any window)
    }
    int x = v;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      before += w < wid ? wsum[w] : 0;
      total += wsum[w];
    }
    if (b < a.bs) a.vis[b] = carry + before + x - v;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) a.vis[a.bs] = carry;
}

// Partial-state slot of request b's piece of chunk c: every chunk holds at
// most two pieces of requests that span several chunks (its first and its
// last), so slot 2c is the piece that starts at the chunk start and 2c + 1
// the one that starts inside it.
__device__ __forceinline__ int64_t piece_slot(int c, int v0, int chunk) {
  return 2 * (int64_t)c + ((int64_t)c * chunk < v0 ? 1 : 0);
}

template <int LQ, int LV, bool VK, int NW, int NS, bool CAP>
__global__ __launch_bounds__((DecCfg<LQ, LV, VK, NW, NS>::NT), 1) void decode_kernel(DecodeArgs a) {
  using C = DecCfg<LQ, LV, VK, NW, NS>;
  constexpr int NDB = LV / 16;  // 16-column output blocks
  constexpr int NKK = LQ / 32;  // 32-dim slices of a K row
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gh = blockIdx.x, c = blockIdx.y;
  const int g = gh / a.hblocks, hb = gh % a.hblocks;
  const int G = a.group;
  const int total = a.vis[a.bs];
  const int cs = c * a.chunk;
  if (cs >= total) return;
  const int ce = min(cs + a.chunk, total);

  // the last request whose visible keys start at or before the chunk start,
  // by a 64-way search: vis[lo] <= cs always holds (vis[0] = 0); each round
  // the lanes probe 64 evenly spaced requests of (lo, hi] at once and the
  // interval shrinks to one step (one memory round trip for up to 65
  // requests, where halving took one per halving)
  int lo = 0, hi = a.bs - 1;
  while (lo < hi) {
    const int step = (hi - lo + 63) >> 6;
    const int p = lo + (lane + 1) * step;
    const bool le = p <= hi && a.vis[p] <= cs;  // true on a prefix of the lanes
    const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
    hi = min(hi, lo + (k + 1) * step - 1);
    lo += k * step;
  }

  char* wbase = lds + w * C::WAVE_BYTES;
  char* ring = wbase + NS * C::STAGE;
  const unsigned r16 = lane & 15;   // K row of this lane's operand reads; also its head row
  const unsigned j4 = lane >> 4;    // lane group: keys 4 j4 .. 4 j4 + 3 of a tile
  const int hrow = hb * 16 + (int)r16;
  const bool hvalid = hrow < G;
  const int head = g * G + hrow;

  for (int b = lo; b < a.bs; ++b) {
    const int v0 = a.vis[b], v1 = a.vis[b + 1];
    if (v0 >= ce) break;
    if (v1 <= v0) continue;
    const int ps = max(cs, v0), pe = min(ce, v1);
    const int kvs = a.kv_indptr[b];
    const int first = (a.kv_indptr[b + 1] - kvs) - (v1 - v0);  // first visible key of b
    const int k_lo = first + (ps - v0), k_hi = first + (pe - v0);
    const int per = ((k_hi - k_lo + NW * kTile - 1) / (NW * kTile)) * kTile;
    const int k0 = min(k_lo + w * per, k_hi), k1 = min(k0 + per, k_hi);
    const int nk = k1 - k0, nt = (nk + kTile - 1) / kTile;

    float m = -INFINITY, lsum = 0.0f;
    f32x4 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nt > 0) {
      // Q^T operand: lane = (head row r16, dims 8 (4 kk + j4) .. + 8)
      bf16x8 qv[NKK];
      {
        const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) + (int64_t)b * a.q_st + (int64_t)head * a.q_sh;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          if (hvalid) {
            qv[kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * j4);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[kk][e] = (__bf16)0.0f;
          }
        }
      }
      const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (int64_t)g * a.kp_sh;
      const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (int64_t)g * a.vp_sh;
      const gptr<char> islots = (gptr<char>)(a.kv_indices + kvs);

      // slot table of tile t (keys past the share repeat its last key)
      auto issue_slots = [&](int t) {
        const int key = min(k0 + kTile * t + (int)((lane >> 1) & 15), k1 - 1);
        load_lds_4(islots + (int64_t)key * 8 + 4 * (lane & 1), lds_addr(ring + (t % C::NSI) * C::SLOT_BYTES));
      };
      // K (and V) rows of tile t into its stage: load i puts lane L's 16 bytes
      // at LDS chunk 64 i + L of the stage, row (64 i + L) / CK
      auto issue_tile = [&](int t) {
        const int64_t* sl = reinterpret_cast<const int64_t*>(ring + (t % C::NSI) * C::SLOT_BYTES);
        char* st = wbase + (t % NS) * C::STAGE;
        auto ksrc = [&](int i) {
          const unsigned f = 64u * i + lane, r = f / C::CK, p = f % C::CK;
          return kbase + sl[r] * a.kp_ss + (p ^ swz_k<C::CK>(r)) * 16u;
        };
        auto vsrc = [&](int i) {
          const unsigned f = 64u * i + lane, r = f / C::CV, p = f % C::CV;
          return vbase + sl[r] * a.vp_ss + (p ^ swz_v<C::CV>(r)) * 16u;
        };
        if constexpr (C::K_LOADS + C::V_LOADS <= 18) {
          // every row address first (one wait for the slot reads), then the loads
          const char* ks[C::K_LOADS];
          const char* vs[C::V_LOADS > 0 ? C::V_LOADS : 1];
#pragma unroll
          for (int i = 0; i < C::K_LOADS; ++i) ks[i] = ksrc(i);
#pragma unroll
          for (int i = 0; i < C::V_LOADS; ++i) vs[i] = vsrc(i);
#pragma unroll
          for (int i = 0; i < C::K_LOADS; ++i) load_lds_16((gptr<void>)ks[i], lds_addr(st + 1024 * i));
#pragma unroll
          for (int i = 0; i < C::V_LOADS; ++i) load_lds_16((gptr<void>)vs[i], lds_addr(st + C::K_BYTES + 1024 * i));
        } else {
          // (too many loads to hold every address in registers)
#pragma unroll
          for (int i = 0; i < C::K_LOADS; ++i) load_lds_16((gptr<void>)ksrc(i), lds_addr(st + 1024 * i));
#pragma unroll
          for (int i = 0; i < C::V_LOADS; ++i) load_lds_16((gptr<void>)vsrc(i), lds_addr(st + C::K_BYTES + 1024 * i));
        }
      };

      // prologue: slot tables 0 .. NS-1, then tiles 0 .. NS-2 each followed by
      // the slot table NS tiles later (the order every later trip keeps)
#pragma unroll
      for (int t = 0; t < NS; ++t) issue_slots(t);
      wait_all_mem();
#pragma unroll
      for (int t = 0; t < NS - 1; ++t) {
        if (t < nt) issue_tile(t);
        issue_slots(t + NS);
      }

      for (int t = 0; t < nt; ++t) {
        // Trip t first refills the stage trip t - 1 has finished with (the
        // wait is also the compiler fence that keeps that trip's operand
        // reads ahead of the refill): tile t + NS - 1, whose slot table has
        // landed once at most the NS - 1 trips issued after it are in flight,
        // then the slot table NS tiles later.  Only then does it wait for
        // tile t, so that while it waits all NS stages are in flight.
        if (t + NS - 1 < nt) {
          wait_vm<C::W_SLOTS>();
          issue_tile(t + NS - 1);
        }
        issue_slots(t + 2 * NS - 1);
        if (t + NS - 1 < nt) wait_vm<C::W_TILE>(); else wait_all_mem();

        const char* st = wbase + (t % NS) * C::STAGE;
        // S^T = K Q^T: lane holds keys 4 j4 .. 4 j4 + 3 of head row r16
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const unsigned cc = 4u * kk + j4;
          const bf16x8 kv = *(lptr<bf16x8>)(st + r16 * (C::CK * 16) + (cc ^ swz_k<C::CK>(r16)) * 16u);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[kk], s, 0, 0, 0);
        }
        // Schedule: the first PRE operand reads, then one product per further
        // read, so that reads stay in flight ahead of the products (left to
        // itself the compiler reused one register and waited for each read
        // before its product: 18 LDS round trips per tile on 576-wide rows).
        // The scheduling barrier after the groups keeps the softmax and the
        // V^T reads out of them.
        {
          constexpr int PRE = NKK < 6 ? NKK : 6;
          __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);  // DS reads
#pragma unroll
          for (int i = 0; i < NKK - PRE; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        float x[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float y;
          if constexpr (CAP) {
            // cap * tanh(scale s / cap) in base-2 units; tanh(u) = 1 - 2 / (e^{2u} + 1)
            const float u = s[i] * a.cap_in;
            y = a.cap_out * (1.0f - 2.0f / (fast_exp2(2.0f * kLog2e * u) + 1.0f));
          } else {
            y = s[i] * a.scale_log2;
          }
          x[i] = kTile * t + 4 * (int)j4 + i < nk ? y : -INFINITY;
          mx = fmaxf(mx, x[i]);
        }
        mx = xor_max(xor_max(mx, 16), 32);
        // the reference max m is raised (and the state rescaled) only when a
        // head's tile max exceeds it by more than 2^8: weights stay <= 2^8
        const bool raise = mx > m + kRescaleSlack;  // always on the first tile (m = -inf)
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          const float m_new = raise ? mx : m;
          const float alpha = fast_exp2(m - m_new);  // 1 for heads that keep m, 0 from m = -inf
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[db] = acc[db] * alpha;
          m = m_new;
        }
        bf16x4 pb;
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = (__bf16)fast_exp2(x[i] - m);
          psum += (float)pb[i];  // the sum adds the rounded weights that multiply V
        }
        lsum += psum;
        const i16x4 pbi = __builtin_bit_cast(i16x4, pb);
        // O^T += V^T P^T: lane (in its group of 16) t16 reads row 4 j4 + t16 / 4 at
        // column 16 db + 4 (t16 % 4) and receives column 16 db + t16 of rows 4 j4 ..
        const unsigned vr = 4u * j4 + (r16 >> 2);
        const unsigned half8 = 8u * (lane & 1);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const unsigned vc = 2u * db + ((lane & 3) >> 1);
          const char* addr;
          if constexpr (VK) {
            addr = st + vr * (C::CK * 16) + (vc ^ swz_k<C::CK>(vr)) * 16u + half8;
          } else {
            addr = st + C::K_BYTES + vr * (C::CV * 16) + (vc ^ swz_v<C::CV>(vr)) * 16u + half8;
          }
          const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr<i16x4>)(addr));
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pbi, acc[db], 0, 0, 0);
        }
      }
      wait_all_mem();  // the slot tables requested past the last tile
    }
    lsum = xor_sum(xor_sum(lsum, 16), 32);

    // ---- merge the waves' states through LDS (the stages are free now)
    barrier_fence();
    float* mml = reinterpret_cast<float*>(lds);              // [NW][16][2]
    float* macc = reinterpret_cast<float*>(lds) + NW * 32;   // [NW][16][MP]
    if (lane < 16) {
      mml[(w * 16 + lane) * 2] = m;
      mml[(w * 16 + lane) * 2 + 1] = lsum;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<float4*>(macc + (w * 16 + r16) * C::MP + 16 * db + 4 * j4) =
          make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
    barrier_fence();

    const int c0 = v0 / a.chunk, c1 = (v1 - 1) / a.chunk;
    const bool single = c0 == c1;
    const int64_t slot = piece_slot(c, v0, a.chunk);
    constexpr int V4 = LV / 4;
    static_assert(16 * V4 % C::NT == 0, "merge items per thread");
    // unrolled by two, so that the LDS reads of two items are issued
    // together (more would spill the 576-wide rows' registers)
#pragma unroll 2
    for (int it = 0; it < 16 * V4 / C::NT; ++it) {
      const int idx = tid + it * C::NT;
      const int row = idx / V4, d = 4 * (idx % V4);
      if (hb * 16 + row >= G) continue;
      float M = -INFINITY;
#pragma unroll
      for (int u = 0; u < NW; ++u) M = fmaxf(M, mml[(u * 16 + row) * 2]);
      float L = 0.0f;
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        const float mu = mml[(u * 16 + row) * 2];
        const float wt = mu == -INFINITY ? 0.0f : fast_exp2(mu - M);
        L += mml[(u * 16 + row) * 2 + 1] * wt;
        const float4 v = *reinterpret_cast<const float4*>(macc + (u * 16 + row) * C::MP + d);
        o.x += v.x * wt;
        o.y += v.y * wt;
        o.z += v.z * wt;
        o.w += v.w * wt;
      }
      const int h = g * G + hb * 16 + row;
      if (single) {
        if (a.sinks) L += fast_exp2(a.sinks[h] * kLog2e - M);
        const float inv = 1.0f / L;
        bf16x4 ov;
        ov[0] = (__bf16)(o.x * inv);
        ov[1] = (__bf16)(o.y * inv);
        ov[2] = (__bf16)(o.z * inv);
        ov[3] = (__bf16)(o.w * inv);
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + (int64_t)b * a.o_st + (int64_t)h * a.o_sh + d) = ov;
      } else {
        const int64_t prow = (slot * a.gh_count + gh) * 16 + row;
        *reinterpret_cast<float4*>(a.part_acc + prow * LV + d) = o;
        if (d == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(M, L);
      }
    }

    barrier_fence();  // the merge area is the next piece's stages
  }
}

// Requests whose keys span several chunks: one workgroup per (head block,
// 64-column slice, request) combines the chunks' states in chunk order
// (deterministic), batch by batch:
//   M = max_c m_c,  L = sum_c l_c 2^(m_c - M),  o = sum_c acc_c 2^(m_c - M) / L
// plus the sink term.  Thread = (head row, 4 columns), the partial rows of
// kMergeBatch chunks in flight per thread at once (one pass: a maximum
// taken first over every chunk would cost a dependent round trip).  A
// request with no visible key gets a zero output here (there is nothing to
// average).
constexpr int kMergeCols = 64;
constexpr int kMergeBatch = 16;

template <int LV>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int SLICES = LV / kMergeCols;
  const int gh = blockIdx.x / SLICES, slice = blockIdx.x % SLICES, b = blockIdx.y;
  const int g = gh / a.hblocks, hb = gh % a.hblocks, G = a.group;
  const int row = threadIdx.x / (kMergeCols / 4), d = slice * kMergeCols + 4 * (threadIdx.x % (kMergeCols / 4));
  if (hb * 16 + row >= G) return;
  const int h = g * G + hb * 16 + row;
  bf16x4* out = reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + (int64_t)b * a.o_st + (int64_t)h * a.o_sh + d);
  const int v0 = a.vis[b], v1 = a.vis[b + 1];
  if (v1 <= v0) {
    *out = bf16x4{(__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
    return;
  }
  const int c0 = v0 / a.chunk, c1 = (v1 - 1) / a.chunk;
  if (c0 == c1) return;  // written by its only chunk
  // the chunks in batches, every load of a batch in flight at once; the
  // running state is rescaled when a batch raises the maximum
  float M = -INFINITY, L = 0.0f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int cb = c0; cb <= c1; cb += kMergeBatch) {
    float2 ml[kMergeBatch];
    float4 v[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      ml[i] = make_float2(-INFINITY, 0.0f);
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (cb + i <= c1) {
        const int64_t prow = (piece_slot(cb + i, v0, a.chunk) * a.gh_count + gh) * 16 + row;
        ml[i] = *reinterpret_cast<const float2*>(a.part_ml + prow * 2);
        v[i] = *reinterpret_cast<const float4*>(a.part_acc + prow * LV + d);
      }
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) Mb = fmaxf(Mb, ml[i].x);
    if (Mb > M) {
      const float sc = M == -INFINITY ? 0.0f : fast_exp2(M - Mb);
      L *= sc;
      o.x *= sc;
      o.y *= sc;
      o.z *= sc;
      o.w *= sc;
      M = Mb;
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const float wt = ml[i].x == -INFINITY ? 0.0f : fast_exp2(ml[i].x - M);
      L += ml[i].y * wt;
      o.x += v[i].x * wt;
      o.y += v[i].y * wt;
      o.z += v[i].z * wt;
      o.w += v[i].w * wt;
    }
  }
  if (a.sinks) L += fast_exp2(a.sinks[h] * kLog2e - M);
  const float inv = 1.0f / L;
  bf16x4 ov;
  ov[0] = (__bf16)(o.x * inv);
  ov[1] = (__bf16)(o.y * inv);
  ov[2] = (__bf16)(o.z * inv);
  ov[3] = (__bf16)(o.w * inv);
  *out = ov;
}

template <int LQ, int LV, bool VK, int NW, int NS>
hipError_t launch_decode_t(const DecodeArgs& a, int64_t chunks, hipStream_t s) {
  if (chunks > 0) {  // (no visible key at all: only the zero outputs of the merge launch)
    const dim3 grid((unsigned)a.gh_count, (unsigned)chunks), block(DecCfg<LQ, LV, VK, NW, NS>::NT);
    if (a.use_cap)
      hipLaunchKernelGGL((decode_kernel<LQ, LV, VK, NW, NS, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<LQ, LV, VK, NW, NS, false>), grid, block, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  static_assert(LV % kMergeCols == 0, "merge slices");
  hipLaunchKernelGGL(decode_merge_kernel<LV>, dim3((unsigned)(a.gh_count * (LV / kMergeCols)), (unsigned)a.bs),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

// bf16 variants: (lq, lv, V inside K, waves per workgroup, LDS stages per wave)
#define PKV_DEC_VARIANTS(X)      \
  X(64, 64, false, 4, 6)         \
  X(128, 128, false, 4, 4)       \
  X(256, 256, false, 4, 2)       \
  X(192, 128, false, 4, 3)       \
  X(288, 256, false, 4, 2)       \
  X(576, 512, true, 4, 2)        \
  X(576, 512, false, 2, 2)

// fp32 decode runs as the unified extend of one new token per request whose
// prefix is every earlier key: these two kernels write its row arrays and
// give requests without keys their zero output afterwards.
__global__ __launch_bounds__(256) void decode_rows_kernel(const int32_t* kv_indptr, int32_t bs, int32_t* qo_indptr,
                                                           int32_t* prefix_lens) {
  for (int b = blockIdx.x * 256 + threadIdx.x; b <= bs; b += gridDim.x * 256) {
    qo_indptr[b] = b;
    if (b < bs) prefix_lens[b] = max(kv_indptr[b + 1] - kv_indptr[b] - 1, 0);
  }
}
__global__ __launch_bounds__(256) void decode_zero_empty_kernel(const int32_t* kv_indptr, int32_t hq, int32_t lv,
                                                                 int32_t elem_bytes, char* o, int64_t o_st,
                                                                 int64_t o_sh) {
  const int b = blockIdx.x;
  if (kv_indptr[b + 1] != kv_indptr[b]) return;
  for (int i = threadIdx.x; i < hq * lv; i += 256) {
    char* e = o + ((int64_t)b * o_st + (int64_t)(i / lv) * o_sh + i % lv) * elem_bytes;
    if (elem_bytes == 4) *reinterpret_cast<float*>(e) = 0.0f;
    else *reinterpret_cast<uint16_t*>(e) = 0;
  }
}

}  // namespace

hipError_t launch_decode_rows(const int32_t* kv_indptr, int32_t bs, int32_t* qo_indptr, int32_t* prefix_lens,
                              hipStream_t s) {
  const unsigned grid = (unsigned)((bs + 1 + 255) / 256 < 1024 ? (bs + 1 + 255) / 256 : 1024);
  hipLaunchKernelGGL(decode_rows_kernel, dim3(grid), dim3(256), 0, s, kv_indptr, bs, qo_indptr, prefix_lens);
  return hipGetLastError();
}

hipError_t launch_decode_zero_empty(const int32_t* kv_indptr, int32_t bs, int32_t hq, int32_t lv, int32_t elem_bytes,
                                    void* o, int64_t o_st, int64_t o_sh, hipStream_t s) {
  if (bs <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_zero_empty_kernel, dim3((unsigned)bs), dim3(256), 0, s, kv_indptr, hq, lv, elem_bytes,
                     static_cast<char*>(o), o_st, o_sh);
  return hipGetLastError();
}

bool decode_supported(int dtype, int lq, int lv, bool v_in_k, int* waves) {
  if (dtype != 0) return false;
#define PKV_DS(Q, V, VK, NW, NS)                  \
  if (lq == Q && lv == V && VK == v_in_k) {       \
    *waves = NW;                                  \
    return true;                                  \
  }
  PKV_DEC_VARIANTS(PKV_DS)
#undef PKV_DS
  return false;
}

hipError_t launch_decode(int lq, int lv, bool v_in_k, const DecodeArgs& a, int64_t chunks, hipStream_t s,
                         hipEvent_t before, hipEvent_t after) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (before && (e = hipEventRecord(before, s)) != hipSuccess) return e;
  e = hipErrorInvalidValue;
#define PKV_DL(Q, V, VK, NW, NS) \
  if (lq == Q && lv == V && VK == v_in_k) e = launch_decode_t<Q, V, VK, NW, NS>(a, chunks, s);
  PKV_DEC_VARIANTS(PKV_DL)
#undef PKV_DL
  if (e == hipSuccess && after) e = hipEventRecord(after, s);
  return e;
}

}  // namespace pkv
