// Extend-attention kernel for bf16 head dims 64, 128, 256 and the 576/512
// latent+rope layout on gfx950, with K/V tiles loaded straight from global
// memory into LDS.
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
//    per tile instead of two.
//  * NS LDS stages: tile t+NS-1 is requested while tile t is computed, deep
//    enough to cover the latency of a gather from the pool under load.  The
//    row slots (kv_indices) of later tiles come into LDS the same way, so the
//    only memory traffic in the loop is these loads, every trip has the same
//    number of them, and the wait at the top of a trip is a fixed vmcnt.
//  * The load places lane L's 16 bytes at base + 16 L, so rows cannot be
//    padded; instead the 16-byte chunk index is XOR-swizzled per row (applied
//    when choosing each lane's global address, undone on reads): the
//    MFMA operand reads of K and the transposing reads of V stay free of bank
//    conflicts.
//  * Head dims 128 and 256 run 256 rows (8 waves, two per SIMD) per
//    workgroup, so one K/V tile in LDS serves twice the rows of a 128-row
//    workgroup.  At 128, waves 0-3 request the next tile's K rows after each
//    barrier and waves 4-7 its V rows after their QK products (waves w and
//    w+4 share a SIMD).  At 256 a wave holds all of its 32 rows' Q^T (64
//    registers) and O^T (128) and takes 32-key tiles in three stages; one
//    half of the waves issues each tile's loads (the half without rows when
//    the item leaves one).
//  * When V is the first Lv columns of K (the MLA layout on page
//    "cpu_graph_runner.py", qkv_proj_with_rope: v = k.narrow(-1, 0, lv)), only
//    the K tile is loaded and the V^T operand is read from it; the Q rows of
//    those 576-wide rows are staged through LDS with whole 1 KB loads.
//  * A workgroup's start requests its first tables' slots before its Q rows
//    and its first tile while they arrive; its end writes 16 bytes of
//    output per lane.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <int LQ, int LV, int BN, bool VK, int RG_, int SPLIT_, int NS_, int DR_ = 0>
struct DlCfg {
  // Plain head dims that are not a served tile width (80, 96, 112 in the
  // 128-wide tile, 160 and 192 in the 256-wide one): the tile keeps its width
  // and the columns from DR on hold zeros -- Q's in registers, K's and V's
  // loaded from the zero row -- so the products over them add nothing; the
  // contraction stops at the last real 16-column step and only output
  // blocks holding real columns are computed and stored (the page's
  // extend kernels pad the head dim to a power of two and mask the columns
  // past Lq the same way: page "extend_attention.py",
  // _get_block_sizes_for_extend_attention and the offs_d < Lq masks).
  static constexpr int LQR = DR_ ? DR_ : LQ;  // real Q/K dims
  static constexpr int LVR = DR_ ? DR_ : LV;  // real V/O dims
  static constexpr int CKR = LQR / 8;         // real 16-byte chunks of a K row
  static constexpr int CVR = LVR / 8;
  // Waves per row group.  When one wave cannot hold both its Q^T operand
  // (LQ / 4 registers) and its O^T accumulator (LV / 2 registers), two waves
  // share a row group: each holds half of the Q dims and half of the O
  // columns, and the two halves of S^T are summed through LDS.  Half h owns
  // chunks 4h..4h+3 of every 8-chunk group of a row (Q/K dims) and the
  // 32-column output blocks 2m + h, so that inside a swizzle group its
  // operand addresses differ from one per-lane base by constants only.
  static constexpr int SPLIT = SPLIT_;
  // 32-row groups per workgroup.  The split variant (576/512) uses 4 (8
  // waves, two per SIMD): a wave's Q^T and O^T halves take ~200 registers,
  // so two waves fit one SIMD's register file.
  static constexpr int RG = RG_;
  // LDS stages: tile kt+NS-1 is requested while tile kt is computed
  static constexpr int NS = NS_;
  static constexpr int NW = RG * SPLIT;
  static constexpr int NT = NW * 64;
  static constexpr int BM = RG * 32;
  static constexpr int QD = LQ / SPLIT;  // Q dims per wave
  static constexpr int VD = LV / SPLIT;  // O columns per wave
  static constexpr int CK = LQ / 8;      // 16-byte chunks per K row
  static constexpr int CV = LV / 8;
  static constexpr int NDB_ALL = LV / 32;  // 32-column output blocks
  // contraction steps and output blocks a wave computes: the split variants
  // interleave the halves inside 8-chunk groups and compute every step
  static constexpr int NQ = SPLIT == 1 ? (CKR + 1) / 2 : QD / 16;
  static constexpr int NDB = SPLIT == 1 ? (LVR + 31) / 32 : VD / 32;
  static constexpr bool WIDE = CK == 72;  // 576-element rows: swizzle inside 8-chunk groups
  // at the register limit (two waves per SIMD, 256 registers each): re-derive
  // the per-lane table and load addresses every trip rather than keep them
  static constexpr bool REMAT = WIDE || LQ >= 256;
  // rows sharing one 256-byte window of the 64 LDS banks
  static constexpr int RPK = CK >= 16 ? 1 : 16 / CK;
  static constexpr int RPV = CV >= 16 ? 1 : 16 / CV;
  static constexpr int SWK = CK >= 16 ? 16 : CK;     // distinct K swizzles
  static constexpr int SWV = CV >= 16 ? 4 : CV / 4;  // distinct V swizzles (multiples of 4 chunks)
  static constexpr int K_BYTES = BN * LQ * 2;
  static constexpr int V_BYTES = VK ? 0 : BN * LV * 2;
  static constexpr int V_PITCH = VK ? LQ * 2 : LV * 2;  // bytes between V rows in LDS
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr int K_CHUNKS = K_BYTES / 1024;  // 1 KB load instructions per tile
  static constexpr int V_CHUNKS = V_BYTES / 1024;
  // per wave; when the chunks do not divide evenly, waves past the last chunk
  // load again a chunk of the last round (same bytes to the same place), so
  // every wave issues the same number of loads
  static constexpr int K_LOADS = (K_CHUNKS + NW - 1) / NW;
  static constexpr int V_LOADS = (V_CHUNKS + NW - 1) / NW;
  // Eight waves (two per SIMD: waves w and w + 4 share one), staggered
  // loads: waves 0..3 issue the K rows of the next tile right after each
  // barrier and waves 4..7 its V rows after their S = K Q^T products, so
  // while one wave of a SIMD waits for the memory pipeline to take its loads,
  // the other has products to run.  Which wave builds the tables is decided
  // per work item (see the kernel).
  static constexpr bool OFFLOAD = SPLIT == 1 && NW == 8 && NS == 2;
  // Eight waves, three stages (head dim 256): one half of the waves issues
  // every load of a tile (each wave its own chunks and those of the wave 4
  // apart) -- waves 0..3 when the item has rows for all eight (the other
  // half of each SIMD then goes straight to its products), waves 4..7 when
  // it leaves them without rows.
  static constexpr bool GROUPED = SPLIT == 1 && NW == 8 && NS == 3;
  static constexpr int LOADERS = OFFLOAD || GROUPED ? NW / 2 : NW;  // waves per load group
  static constexpr int TW = 0;                            // the wave that builds tables (not staggered)
  static constexpr int L = OFFLOAD ? 2 * V_LOADS : K_LOADS + V_LOADS;  // tile loads per wave per tile
  static constexpr int I = BN * 8 / 256;  // row-slot loads (64 lanes x 4 bytes) per tile, table wave
  // waits at the top of an iteration (see the loop): outstanding loads allowed
  static constexpr int W_OTHER = (NS - 2) * L;
  // (the row slots of a tile are requested in the same group as the tile
  // NS-1 groups before it, so the tile's wait is the binding one)
  static constexpr int W_TABLE = (NS - 2) * (I + L);
  // grouped loads: a loading wave issues twice the chunks, the others none
  static constexpr int L_G = 2 * (K_LOADS + V_LOADS);
  static constexpr int W_LOADER_G = (NS - 2) * L_G;
  static constexpr int W_TABLE_G = (NS - 2) * (I + L_G);
  static constexpr int XCH_BYTES = SPLIT > 1 ? NW * BN * 32 * 4 : 0;  // S^T halves exchanged
  // 576-wide rows: the workgroup's Q rows staged through LDS at the start
  // (laid out like a K tile), in the space of the stages
  static constexpr int QST_BYTES = WIDE ? BM * LQ * 2 : 0;
  static constexpr int LDS_BYTES = NS * STAGE_BYTES + XCH_BYTES > QST_BYTES ? NS * STAGE_BYTES + XCH_BYTES : QST_BYTES;
  static_assert(QST_BYTES % (1024 * NW) == 0, "Q staging: whole 1 KB loads, the same count per wave");
  static_assert(CK == 8 || CK == 16 || CK == 32 || CK == 72, "lq");
  static_assert(VK ? LV <= LQ : (CV == 8 || CV == 16 || CV == 32), "lv");
  static_assert(!WIDE || VK, "576-wide rows only with V inside K");
  static_assert(K_CHUNKS >= NW && (V_CHUNKS == 0 || V_CHUNKS >= NW), "every wave has a chunk to repeat");
  static_assert(NS >= 2 && NS <= 5 && W_TABLE < 64 && W_OTHER < 64 && W_TABLE_G < 64, "pipeline depth (slot ring of 4)");
  static_assert(!OFFLOAD || (NS == 2 && K_LOADS == V_LOADS), "staggered loads: every wait is vmcnt(0)");
  static_assert(RG >= 2 || SPLIT == 1, "split variant: at least two row groups");
  static_assert(QD % 16 == 0 && VD % 32 == 0, "split");
  static_assert(SPLIT == 1 || (SPLIT == 2 && CK % 8 == 0 && NDB_ALL % 2 == 0), "split: halves interleave in 8-chunk groups");
  static_assert(BN % 32 == 0 && BN <= 128, "key tile");
  static_assert(DR_ == 0 || (!VK && LQ == LV && DR_ < LQ && DR_ % 16 == 0), "padded plain head dims");
};

// Physical 16-byte chunk of logical chunk c in row r.  K: the 32 rows read at
// one logical chunk by an MFMA operand load spread over all 16 bank groups.
// V: the 4 rows x 4 chunks of one transposing read spread over all 16 groups.
// 576-wide rows (72 chunks, pitch = 8 groups mod 16): the XOR stays inside
// each group of 8 chunks, g(s) = 4 (s & 1) + (s >> 1) over s = (r / 2) % 8,
// which satisfies both read patterns on the one tile that holds K and V.
__device__ __forceinline__ int wide_xor(int r) {
  const int s = (r >> 1) & 7;
  return ((s & 1) << 2) | (s >> 1);
}
// (r and c are never negative; unsigned arithmetic keeps the divisions shifts)
template <class C>
__device__ __forceinline__ int swz_k(int r, int c) {
  const unsigned ur = r, uc = c;
  if constexpr (C::WIDE) {
    return (int)((uc & ~7u) | ((uc & 7u) ^ (unsigned)wide_xor(r)));
  } else {
    return (int)(uc ^ ((ur / C::RPK) % C::SWK));
  }
}
template <class C>
__device__ __forceinline__ int swz_v(int r, int c) {
  const unsigned ur = r, uc = c;
  if constexpr (C::WIDE) {
    return swz_k<C>(r, c);
  } else {
    return (int)(uc ^ (4u * ((ur / C::RPV) % C::SWV)));
  }
}

// OPT: a sliding window or a custom mask (which replaces the causal rule) may
// be set -- a variant of its own, so that calls without them run code that
// holds no register for them
template <int LQ, int LV, int BN, bool VK, int RG, int SP, int NS, int DR, bool CAP, bool OPT, int MINB>
__global__ __launch_bounds__((DlCfg<LQ, LV, BN, VK, RG, SP, NS, DR>::NT), MINB) void attn_dl_kernel(AttnArgs a) {
  using C = DlCfg<LQ, LV, BN, VK, RG, SP, NS, DR>;
  using T = uint16_t;
  constexpr int BM = C::BM;
  constexpr int NKB = BN / 32;
  constexpr int NQ = C::NQ;
  constexpr int NDB = C::NDB;

  __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];
  __shared__ gptr<T> kptr[NS][BN];  // row pointer tables, slot kt % NS
  __shared__ gptr<T> vptr[NS][BN];
  __shared__ __attribute__((aligned(16))) int64_t slots[4][BN];  // row slots of later tiles, slot kt & 3

  // the work record and the plan header in one round trip: the grid is the
  // workspace's capacity of records, so every block index names a record.
  // (Left alone, the compiler loads each piece right before its first use,
  // one round trip after another; the empty asm takes a field of every 16
  // bytes and the header before the branch.)
  const WorkItem it = a.work[blockIdx.x];
  const int num_work = a.hdr->num_work;
  asm volatile("" ::"s"(it.b), "s"(it.kt_end), "s"(it.q0), "s"(it.n_idx), "s"(num_work));
  if (it.b < 0 || (int)blockIdx.x >= num_work) return;  // empty or unused placement slot
  const int tid = threadIdx.x, lane = tid & 63;
  // the lane index the loop's table and load addressing starts from: the
  // variants at their register limit (REMAT, and those with options)
  // re-derive those per-lane addresses on every trip from this copy (see the
  // loop) -- a few VALU operations -- where the compiler would otherwise keep
  // them across the loop and spill them
  int ln = lane;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
  const int rg = wv % C::RG, half = wv / C::RG;  // row group; which half of Q dims / O columns
  const int qi = lane & 31, hi = lane >> 5;
  // first 16-byte chunk of contraction step ks (its lanes hi = 0, 1 take ch, ch + 1)
  auto qk_chunk = [&](int ks) __attribute__((always_inline)) {
    return C::SPLIT > 1 ? 8 * (ks >> 1) + 4 * half + 2 * (ks & 1) : 2 * ks;
  };
  // 32-column output block of this wave's block db
  auto o_block = [&](int db) __attribute__((always_inline)) { return C::SPLIT > 1 ? 2 * db + half : db; };
  const int G = a.group;
  const int b = it.b, g = it.g;
  const bool causal = !OPT || a.custom_mask == nullptr;
  const SeqKeys sk = item_keys(it);
  const int q0 = sk.q0, E = sk.E, kvs = sk.kvs, P = sk.P;
  const int R = E * G;
  // last visible key of a row of token i: the diagonal, or every key with a custom mask
  auto last_key = [&](int i) __attribute__((always_inline)) { return causal ? min(P + i, sk.n_keys - 1) : sk.n_keys - 1; };

  const int r = it.t * BM + rg * 32 + qi;
  const bool valid = r < R;
  const int W = OPT ? a.window : 0;
  const int lim = valid ? last_key(r / G) : -1;  // last visible key of this lane's row
  const int lo = (W > 0 && valid) ? P + r / G - W : kNoLowerKey;  // first visible key (sliding window)
  const int rw0 = it.t * BM + rg * 32;
  const bool wave_live = rw0 < R;
  // the wave's smallest and largest last (lim) and first (lo) visible key
  const int tok_lo_w = wave_live ? rw0 / G : 0, tok_hi_w = wave_live ? min(R - 1, rw0 + 31) / G : 0;
  const int lim_lo_w = last_key(tok_lo_w);
  const int lim_hi_w = last_key(tok_hi_w);
  const int lo_lo_w = W > 0 ? P + tok_lo_w - W : kNoLowerKey;
  const int lo_hi_w = W > 0 ? P + tok_hi_w - W : kNoLowerKey;
  const int key_last = last_key(min(R - 1, it.t * BM + BM - 1) / G);
  // The table wave with staggered loads: a wave without rows when the item
  // leaves the last one empty, else wave 3 -- the waves of the K group
  // finish their tile first and wait at the barrier the longest, while
  // table work on a wave of the V group delays the whole tile.
  const int n_live = min(C::NW, (R - it.t * BM + 31) / 32);  // waves with rows (one row group each when staggered)
  // grouped loads: the loading half of the waves, and its table wave
  const bool upper_loads = C::GROUPED && R - it.t * BM <= (C::RG / 2) * 32;
  const bool loader = !C::GROUPED || (upper_loads ? wv >= C::LOADERS : wv < C::LOADERS);
  const int tw = C::GROUPED ? (upper_loads ? C::NW - 1 : C::TW)
                            : !C::OFFLOAD ? C::TW : n_live < C::NW ? C::NW - 1 : C::LOADERS - 1;

  const gptr<T> kpool = (gptr<T>)a.k_pool;
  const gptr<T> vpool = (gptr<T>)a.v_pool;
  const gptr<T> kext = (gptr<T>)a.k_ext;
  const gptr<T> vext = (gptr<T>)a.v_ext;
  const gptr<T> zrow = (gptr<T>)a.zero_row;
  const int kt0 = it.kt_begin, kt1 = it.kt_end;
  // last key whose K/V rows are loaded: the tiles the pipeline requests past
  // the chunk's range (so that every trip has the same loads in flight) read
  // the zero row, not the next chunk's keys
  const int key_load_last = min(key_last, kt1 * BN - 1);

  // ---- 576-wide rows: the item's Q rows into LDS with whole 1 KB loads, 16
  //      contiguous bytes per lane (loaded into registers directly, one
  //      instruction touches 32 rows' cache lines for 32 bytes each, and on
  //      MLA issuing the 18 per wave took ~8 us), in the K tile's layout:
  //      row-major at 2 LQ bytes a row, chunk c at swz_k(row, c), so that the
  //      operand reads below are those of the QK products
  if constexpr (C::WIDE) {
#pragma unroll
    for (int i = 0; i < C::QST_BYTES / 1024 / C::NW; ++i) {
      const unsigned pos = (unsigned)(i * C::NW + wv) * 64u + (unsigned)lane;  // 16-byte slot of this lane
      const unsigned row = pos / C::CK;
      const int cl = swz_k<C>((int)row, (int)(pos % C::CK));  // the logical chunk stored there
      const int ri = it.t * BM + (int)row;
      gptr<T> src = zrow + cl * 8;  // rows past the item: zeros
      if (ri < R) src = (gptr<T>)a.q + (int64_t)(q0 + ri / G) * a.q_st + (int64_t)(g * G + ri % G) * a.q_sh + cl * 8;
      load_lds_16((gptr<void>)src, lds_addr(lds + 1024 * (i * C::NW + wv)));
    }
  }

  // ---- slots of the first NS - 1 tables (waves 0 .. NS - 2 build one each):
  //      from the index array, or the zero row's 8 zero bytes
  constexpr int EPL = (BN + 63) / 64;  // keys per lane
  static_assert(NS - 1 <= C::NW, "one first table per wave at most");
  const bool builds_first = kt0 < kt1 && wv < NS - 1;
  int64_t sl0[EPL];
  if (builds_first) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i, j = (kt0 + wv) * BN + e;
      const bool real = e < BN && j < sk.n_idx && j <= key_load_last;
      sl0[i] = *(real ? (gptr<int64_t>)a.kv_indices + ((int64_t)kvs + j) : (gptr<int64_t>)zrow);
    }
  }

  // ---- row pointer tables (NS slots), built by the table wave tw; lane e owns key kt*BN + e.
  //      Strides and per-head bases are read once into scalar registers.
  const int64_t kp_ss = uniform64(a.kp_ss), vp_ss = uniform64(a.vp_ss);
  const int64_t ke_st = uniform64(a.ke_st), ve_st = uniform64(a.ve_st);
  const gptr<T> kpool_g = kpool + (int64_t)g * uniform64(a.kp_sh);
  const gptr<T> vpool_g = vpool + (int64_t)g * uniform64(a.vp_sh);
  const gptr<T> kext_g = kext + (int64_t)g * uniform64(a.ke_sh);
  const gptr<T> vext_g = vext + (int64_t)g * uniform64(a.ve_sh);
  // pointers of key j (pool slot `slot` when j is a prefix key) for a table
  auto key_ptrs = [&](int j, int64_t slot, gptr<T>& kp, gptr<T>& vp) __attribute__((always_inline)) {
    kp = zrow;
    vp = zrow;
    if (j <= key_load_last) {
      if (j < sk.n_idx) {
        kp = kpool_g + slot * kp_ss;
        vp = vpool_g + slot * vp_ss;
      } else {
        const int64_t row = q0 + (j - P);
        kp = kext_g + row * ke_st;
        vp = vext_g + row * ve_st;
      }
    }
  };
  // table of tile kt from the row slots already in LDS (table wave)
  auto write_table = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int e = ln; e < (BN > 64 ? BN : 64); e += 64) {
      if (e < BN) {
        gptr<T> kp, vp;
        key_ptrs(kt * BN + e, slots[kt & 3][e], kp, vp);
        kptr[kt % NS][e] = kp;
        vptr[kt % NS][e] = vp;
      }
    }
  };
  // row slots of tile kt into LDS (table wave): I loads of 64 lanes x 4 bytes;
  // keys outside the prefix or past the last visible key read the zero row
  auto issue_slots = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::I; ++i) {
      const int o = i * 256 + ln * 4;  // byte offset in the tile's slot block
      const int j = kt * BN + o / 8;
      gptr<char> src = (gptr<char>)zrow;
      if (j < sk.n_idx && j <= key_load_last) src = (gptr<char>)a.kv_indices + (int64_t)(kvs + j) * 8 + (o & 4);
      load_lds_4((gptr<void>)src, lds_addr(&slots[kt & 3][0]) + i * 256);
    }
  };

  // ---- direct loads of tile kt into stage kt % NS: wave w covers bytes
  //      [(i * NW + w) * 1024, +1024) of the K and V regions
  // 1 KB chunk of load i of wave w (a chunk of the last round again past the end)
  auto kchunk = [&](int i, int w) __attribute__((always_inline)) {
    const int li = i * C::NW + w;
    return li < C::K_CHUNKS ? li : li - C::NW;
  };
  auto vchunk = [&](int i, int w) __attribute__((always_inline)) {
    const int li = i * C::NW + w;
    return li < C::V_CHUNKS ? li : li - C::NW;
  };
  // K rows (do_k) and V rows (do_v) of tile kt; with staggered loads a wave
  // of either group covers the chunks of two waves (itself and 4 apart)
  auto issue_loads = [&](int kt, bool do_k, bool do_v) __attribute__((always_inline)) {
    constexpr int PER = C::NW / C::LOADERS;  // chunk sets per wave
    const uint32_t stage = lds_addr(lds + (kt % NS) * C::STAGE_BYTES);
    gptr<T> ksrc[PER][C::K_LOADS];
    gptr<T> vsrc[PER][C::V_LOADS > 0 ? C::V_LOADS : 1];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int vw = C::OFFLOAD || C::GROUPED ? wv % C::LOADERS + q * C::LOADERS : wv;  // wave whose chunks these are
      if (do_k) {
#pragma unroll
        for (int i = 0; i < C::K_LOADS; ++i) {
          const unsigned off = (unsigned)kchunk(i, vw) * 1024u + (unsigned)ln * 16u;
          const unsigned row = off / (LQ * 2), p = (off % (LQ * 2)) / 16;
          const unsigned c = (unsigned)swz_k<C>(row, p);
          ksrc[q][i] = C::CKR < C::CK && c >= (unsigned)C::CKR ? zrow : kptr[kt % NS][row] + c * 8u;
        }
      }
      if (do_v) {
#pragma unroll
        for (int i = 0; i < C::V_LOADS; ++i) {
          const unsigned off = (unsigned)vchunk(i, vw) * 1024u + (unsigned)ln * 16u;
          const unsigned row = off / (LV * 2), p = (off % (LV * 2)) / 16;
          const unsigned c = (unsigned)swz_v<C>(row, p);
          vsrc[q][i] = C::CVR < C::CV && c >= (unsigned)C::CVR ? zrow : vptr[kt % NS][row] + c * 8u;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int vw = C::OFFLOAD || C::GROUPED ? wv % C::LOADERS + q * C::LOADERS : wv;
      if (do_k) {
#pragma unroll
        for (int i = 0; i < C::K_LOADS; ++i) load_lds_16((gptr<void>)ksrc[q][i], stage + kchunk(i, vw) * 1024);
      }
      if (do_v) {
#pragma unroll
        for (int i = 0; i < C::V_LOADS; ++i)
          load_lds_16((gptr<void>)vsrc[q][i], stage + C::K_BYTES + vchunk(i, vw) * 1024);
      }
    }
  };
  // every load of tile kt: K by waves 0..3 and V by waves 4..7 when staggered
  auto issue_tile = [&](int kt) __attribute__((always_inline)) {
    if constexpr (C::OFFLOAD) {
      issue_loads(kt, wv < C::LOADERS, wv >= C::LOADERS);
    } else if constexpr (C::GROUPED) {
      if (loader) issue_loads(kt, true, true);
    } else {
      issue_loads(kt, true, true);
    }
  };

  // wide rows: per-lane byte offsets of the operand reads inside a stage.
  // K: row qi, chunk 4 half + 2 m + hi of a group (m = ks & 1).  V^T: rows
  // key0 + 8 x, chunk 4 half + cofs / 8 of a group; all other rows and
  // groups the wave reads add multiples of 32 rows, 16 rows or 128 bytes,
  // which keep the swizzle.
  int k_lane[2] = {0, 0}, v_lane[2] = {0, 0};
  if constexpr (C::WIDE) {
    const int key0 = 4 * hi + ((lane & 15) >> 2);
    const int cofs = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      k_lane[m] = qi * LQ * 2 + ((4 * half + 2 * m + hi) ^ wide_xor(qi)) * 16;
      const int vr = key0 + 8 * m;
      v_lane[m] = vr * C::V_PITCH + ((4 * half + cofs / 8) ^ wide_xor(vr)) * 16 + (cofs % 8) * 2;
    }
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_ref = -INFINITY;  // reference max of the exponentials, base-2 units
  float l_run = 0.0f;       // this lane's share of the running sum

  // Pipeline.  Iteration kt computes tile kt while tiles kt+1 .. kt+NS-2 are
  // in flight; after its barrier it requests the row slots of tile kt+2NS-2
  // (table wave) and then tile kt+NS-1: a tile's slots get as many groups of
  // lead as its rows (NS-1), so deeper stages deepen both.  Tiles and slots past the end of the
  // range are requested too (zero rows, unused), so every wave has the same
  // number of loads in flight on every trip and the waits are fixed counts.

  // the first NS - 1 tables from their slots (the only loads in flight yet)
  if (builds_first) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (e < BN) {
        gptr<T> kp, vp;
        key_ptrs((kt0 + wv) * BN + e, sl0[i], kp, vp);
        kptr[(kt0 + wv) % NS][e] = kp;
        vptr[(kt0 + wv) % NS][e] = vp;
      }
    }
  }

  // ---- Q^T operand (B) in registers, negated when the scale is negative
  //      (requested after the first tables, so that those wait only for
  //      their slots and the Q rows arrive while tile kt0 is in flight)
  bf16x8 qr[NQ];
  if constexpr (C::WIDE) {
    // from the staged rows, once every wave's loads (and the table slots)
    // have landed; a second barrier frees the staging space for the tiles
    wait_all_mem();
    barrier_fence();
    const uint32_t flip = a.neg_q ? 0x80008000u : 0u;
    const char* qs = lds + rg * 32 * LQ * 2;
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
      const int ch = qk_chunk(ks) + hi;
      const u32x4 v = *reinterpret_cast<const u32x4*>(qs + qi * LQ * 2 + swz_k<C>(qi, ch) * 16);
      qr[ks] = valid ? __builtin_bit_cast(bf16x8, v ^ flip) : bf16x8{};
    }
    wait_lds();
    barrier_fence();
  } else {
    const uint32_t flip = a.neg_q ? 0x80008000u : 0u;
    gptr<T> qrow = (gptr<T>)a.q + (int64_t)(q0 + (valid ? r / G : 0)) * a.q_st +
                   (int64_t)(g * G + (valid ? r % G : 0)) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
      const int ch = qk_chunk(ks) + hi;
      const u32x4 v = valid && ch < C::CKR ? *(gptr<u32x4>)(qrow + ch * 8) : u32x4{0u, 0u, 0u, 0u};
      qr[ks] = __builtin_bit_cast(bf16x8, v ^ flip);
    }
  }

  if (kt0 < kt1) {
    // the tables published by a barrier that does not wait for the Q rows
    // (576-wide rows: the barriers above did)
    if constexpr (!C::WIDE) {
      wait_lds();
      barrier_fence();
    }
    // the groups that iterations kt0-NS+1 .. kt0-1 would have issued; tile
    // kt0 goes out while the Q rows are still arriving, and the full wait
    // after it (Q rows, slots, tile kt0) leaves no load the compiler tracks
    // outstanding in the loop
    if (wv == tw) issue_slots(kt0 + NS - 1);
    issue_tile(kt0);
    wait_all_mem();
#pragma unroll
    for (int v = 1; v < NS - 1; ++v) {
      if (wv == tw) issue_slots(kt0 + NS - 1 + v);
      issue_tile(kt0 + v);
    }
  }

  // ---- tile math
  auto active = [&](int kt) __attribute__((always_inline)) {
    return wave_live && kt * BN <= lim_hi_w && kt * BN + BN - 1 >= lo_lo_w;
  };

  // S^T = K Q^T over this wave's Q dims
  auto qk = [&](int kt, f32x16 (&s)[NKB]) __attribute__((always_inline)) {
    const char* Ks = lds + (kt % NS) * C::STAGE_BYTES;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const char* ka;
        if constexpr (C::WIDE) {
          // rows kb*32 + qi share qi's swizzle; the group offset is a constant
          ka = Ks + k_lane[ks & 1] + kb * 32 * LQ * 2 + (ks >> 1) * 128;
        } else {
          const int row = kb * 32 + qi;
          ka = Ks + row * LQ * 2 + swz_k<C>(row, qk_chunk(ks) + hi) * 16;
        }
        const bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ka));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qr[ks], s[kb], 0, 0, 0);
      }
    }
    // Schedule: the first PRE K operand reads, then one product per further
    // read, so PRE - 1 reads stay in flight ahead of the products (left to
    // itself the compiler kept one, and each product waited on LDS latency;
    // eight measured ~7 % faster on llama8b).  Not for the 576-wide rows:
    // with their Q^T and O^T halves the constraint adds spills.
    if constexpr (!C::WIDE) {
      constexpr int PRE = NQ * NKB < 8 ? NQ * NKB : 8;
      __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);  // DS reads
#pragma unroll
      for (int i = 0; i < NQ * NKB - PRE; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
    }
  };

  // split waves: the two halves of S^T meet in LDS; a + b == b + a, so both
  // waves of the pair hold the same S^T bit for bit and take the same
  // softmax decisions.  Contains a barrier: every wave calls it.  The buffer
  // is free again at the next tile's barrier, which every wave reaches only
  // after its reads have returned.
  auto exchange = [&](bool act, f32x16 (&s)[NKB]) __attribute__((always_inline)) {
    f32x4* xw = reinterpret_cast<f32x4*>(lds + NS * C::STAGE_BYTES) + wv * (NKB * 4 * 64);
    const f32x4* xr =
        reinterpret_cast<const f32x4*>(lds + NS * C::STAGE_BYTES) + ((wv + C::RG) % C::NW) * (NKB * 4 * 64);
    if (act) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          xw[(kb * 4 + q4) * 64 + ln] = f32x4{s[kb][4 * q4], s[kb][4 * q4 + 1], s[kb][4 * q4 + 2], s[kb][4 * q4 + 3]};
    }
    wait_lds();
    barrier_fence();
    if (act) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        f32x16 o;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = xr[(kb * 4 + q4) * 64 + ln];
          o[4 * q4] = v[0];
          o[4 * q4 + 1] = v[1];
          o[4 * q4 + 2] = v[2];
          o[4 * q4 + 3] = v[3];
        }
        s[kb] += o;
      }
    }
  };

  // softmax head: soft-cap (base-2 units), mask of the diagonal tiles, row
  // max and lazy rescale; returns the value subtracted in the exponent
  auto softmax_head = [&](int kt, f32x16 (&s)[NKB]) __attribute__((always_inline)) -> float {
    const int j0 = kt * BN;
    const bool need_mask = j0 + BN - 1 > lim_lo_w || j0 < lo_hi_w || !causal;
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
      // custom mask: this row's bytes, key j at mrow[j] (addressed here, inside
      // the branch, so that calls without a mask hold no register for it)
      const uint8_t* mrow = a.custom_mask + a.mask_indptr[b] + (int64_t)(valid ? r / G : 0) * sk.n_keys;
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
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleSlack)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    return m_ref == -INFINITY ? 0.0f : m_ref;
  };
  // P = exp2(s - m) rounded to bf16 in B-operand layout and its row sum
  // (bf16 dot2 with ones); no branches
  auto softmax_exp = [&](const f32x16 (&s)[NKB], float m_sub, bf16x8 (&pb)[NKB][2]) __attribute__((always_inline)) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8 q;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = s[kb][8 * hf + e];
          const float p = CAP ? fast_exp2(x - m_sub) : fast_exp2(fmaf(x, a.scale_log2, -m_sub));
          q[e] = (__bf16)p;
        }
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 0, 1), ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 2, 3), ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 4, 5), ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 6, 7), ones, l_run, false);
        pb[kb][hf] = q;
      }
    }
  };
  auto softmax = [&](int kt, f32x16 (&s)[NKB], bf16x8 (&pb)[NKB][2]) __attribute__((always_inline)) {
    softmax_exp(s, softmax_head(kt, s), pb);
  };

  // O^T += V^T P^T, the V^T operand through transposing LDS reads
  const int key0 = 4 * hi + ((lane & 15) >> 2);
  const int cofs = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto pv = [&](int kt, const bf16x8 (&pb)[NKB][2]) __attribute__((always_inline)) {
    const char* Ks = lds + (kt % NS) * C::STAGE_BYTES;
    const char* Vs = VK ? Ks : Ks + C::K_BYTES;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int r0 = kb * 32 + 16 * hf + key0, r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char *a0, *a1;
          if constexpr (C::WIDE) {
            const int cst = (kb * 32 + 16 * hf) * C::V_PITCH + db * 128;
            a0 = Vs + v_lane[0] + cst;
            a1 = Vs + v_lane[1] + cst;
          } else {
            const int col = o_block(db) * 32 + cofs;
            a0 = Vs + r0 * C::V_PITCH + swz_v<C>(r0, col / 8) * 16 + (col % 8) * 2;
            a1 = Vs + r1 * C::V_PITCH + swz_v<C>(r1, col / 8) * 16 + (col % 8) * 2;
          }
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr<i16x4>)(a0));
          const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr<i16x4>)(a1));
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][hf], acc[db], 0, 0, 0);
        }
      }
    }
  };

  // Top of iteration kt.  Tile kt and the row slots of tile kt+NS-1 were
  // requested NS-1 groups ago (the slots first): wait until at most the later
  // loads are outstanding.  The table wave then writes table kt+NS-1
  // (its slot held table kt-1, issued long ago) before the barrier that
  // publishes it and tile kt.
  auto tile_top = [&](int kt) __attribute__((always_inline)) {
    if (wv == tw) {
      if constexpr (C::GROUPED) wait_vm<C::W_TABLE_G>(); else wait_vm<C::W_TABLE>();
      write_table(kt + NS - 1);
      wait_lds();
    } else if constexpr (C::GROUPED) {
      if (loader) wait_vm<C::W_LOADER_G>(); else wait_vm<0>();
    } else {
      wait_vm<C::W_OTHER>();
    }
    barrier_fence();
  };
  // the group of iteration kt: row slots of tile kt+2NS-2 (table wave; ring
  // entry of tile kt+NS-1, whose table was written before the barrier) and
  // tile kt+NS-1 into stage (kt-1) % NS, which tile kt-1 no longer needs
  auto issue_group = [&](int kt) __attribute__((always_inline)) {
    if (wv == tw) issue_slots(kt + 2 * NS - 2);
    if constexpr (C::OFFLOAD) {
      if (wv < C::LOADERS) issue_loads(kt + NS - 1, true, false);
    } else {
      issue_tile(kt + NS - 1);
    }
  };

  for (int kt = kt0; kt < kt1; ++kt) {
    if constexpr (C::REMAT || OPT) asm volatile("" : "+v"(ln));  // (ln is lane; the compiler no longer knows it)
    tile_top(kt);
    issue_group(kt);
    const bool act = active(kt);
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    if (act) qk(kt, s);
    // staggered loads: the V rows of the tile the group requested
    if constexpr (C::OFFLOAD) {
      if (wv >= C::LOADERS) issue_loads(kt + NS - 1, false, true);
    }
    if constexpr (C::SPLIT > 1) exchange(act, s);
    if (act) {
      bf16x8 pb[NKB][2];
      softmax(kt, s, pb);
      pv(kt, pb);
    }
  }

  // the requests past the end may still be writing LDS
  wait_all_mem();

  // ---- epilogue
  const float l_tot = pair_sum(l_run);
  if (it.part < 0) {
    if (!valid) return;
    // a sink joins the denominator once, here or in the merge of split chunks
    const float inv = 1.0f / (a.sinks ? l_tot + fast_exp2(a.sinks[g * G + r % G] * kLog2e - m_ref) : l_tot);
    T* orow = reinterpret_cast<T*>(a.o) + (int64_t)(q0 + r / G) * a.o_st + (int64_t)(g * G + r % G) * a.o_sh;
    // Lanes hi = 0 and 1 of a row hold dims 8 g4 + 4 hi + (0..3) of each
    // 32-column block; one exchange between them gives each lane 8
    // consecutive dims, 16 h2 + 8 hi + (0..7), written with one 16-byte
    // store (half the store instructions of 8-byte writes, and half the
    // partial cache lines each touches)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int d = o_block(db) * 32 + 16 * h2 + 8 * hi;
        bf16x8 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = acc[db][8 * h2 + j], up = acc[db][8 * h2 + 4 + j];  // dims 16 h2 + 4 hi + j, + 8
          const float got = __shfl_xor(hi ? lo : up, 32);                        // the partner's value this lane needs
          ov[j] = (__bf16)((hi ? got : lo) * inv);
          ov[4 + j] = (__bf16)((hi ? up : got) * inv);
        }
        if (C::LVR < LV && d >= C::LVR) continue;  // padded columns
        *reinterpret_cast<bf16x8*>(orow + d) = ov;
      }
    }
  } else {
    // the merge reads only rows of the item's tokens: padding rows write nothing
    if (!valid) return;
    const int64_t prow = (int64_t)it.part * BM + rg * 32 + qi;
    float* pa = a.part_acc + prow * C::LVR;  // rows of the real width
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = o_block(db) * 32 + 8 * g4 + 4 * hi;
        if (C::LVR < LV && d >= C::LVR) continue;
        *reinterpret_cast<float4*>(pa + d) =
            make_float4(acc[db][4 * g4], acc[db][4 * g4 + 1], acc[db][4 * g4 + 2], acc[db][4 * g4 + 3]);
      }
    }
    if (hi == 0 && half == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(m_ref, l_tot);
  }
}

template <int LQ, int LV, int BN, bool VK, int RG, int SP, int NS, int DR, int MINB>
hipError_t launch_dl_t(const AttnArgs& a, int64_t grid, hipStream_t s) {
  using C = DlCfg<LQ, LV, BN, VK, RG, SP, NS, DR>;
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid), t(C::NT);
  if (a.custom_mask || a.window > 0) {
    if (a.use_cap)
      hipLaunchKernelGGL((attn_dl_kernel<LQ, LV, BN, VK, RG, SP, NS, DR, true, true, MINB>), g, t, 0, s, a);
    else
      hipLaunchKernelGGL((attn_dl_kernel<LQ, LV, BN, VK, RG, SP, NS, DR, false, true, MINB>), g, t, 0, s, a);
  } else if (a.use_cap) {
    hipLaunchKernelGGL((attn_dl_kernel<LQ, LV, BN, VK, RG, SP, NS, DR, true, false, MINB>), g, t, 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_dl_kernel<LQ, LV, BN, VK, RG, SP, NS, DR, false, false, MINB>), g, t, 0, s, a);
  }
  return hipGetLastError();
}

template <int LQ, int LV, int BN, bool VK, int RG, int SP, int NS, int DR, int MINB>
int dl_occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&attn_dl_kernel<LQ, LV, BN, VK, RG, SP, NS, DR, false, false, MINB>),
          DlCfg<LQ, LV, BN, VK, RG, SP, NS, DR>::NT, 0) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

// bf16 variants served here: (lq, lv, key tile, V inside K, 32-row groups,
// waves per row group, LDS stages, real plain head dim in a wider tile or 0,
// workgroups per CU)
// (lq, lv, keys per tile, V inside K, row groups, waves per row group,
//  stages, real plain head dim, min blocks per CU)
#define PKV_DL_VARIANTS(X)                   \
  X(64, 64, 64, false, 4, 1, 4, 0, 2)        \
  X(128, 128, 128, false, 8, 1, 2, 0, 1)     \
  X(256, 256, 32, false, 8, 1, 3, 0, 1)      \
  X(576, 512, 32, true, 4, 2, 3, 0, 1)       \
  X(128, 128, 128, false, 8, 1, 2, 80, 1)    \
  X(128, 128, 128, false, 8, 1, 2, 96, 1)    \
  X(128, 128, 128, false, 8, 1, 2, 112, 1)   \
  X(256, 256, 32, false, 8, 1, 3, 160, 1)    \
  X(256, 256, 32, false, 8, 1, 3, 192, 1)

// head dims a variant serves: its tile's, or the real plain dim it pads
#define PKV_DL_MATCH(Q, V, VK, DR) \
  (lq == ((DR) ? (DR) : (Q)) && lv == ((DR) ? (DR) : (V)) && (!(VK) || v_in_k))

}  // namespace

bool dl_tiling(int dtype, int lq, int lv, bool v_in_k, Tiling* t) {
  if (dtype != 0) return false;
#define PKV_DT(Q, V, N, VK, RG, SP, NS, DR, M)          \
  if (PKV_DL_MATCH(Q, V, VK, DR)) {                     \
    t->bm = DlCfg<Q, V, N, VK, RG, SP, NS, DR>::BM;     \
    t->bn = N;                                          \
    t->threads = DlCfg<Q, V, N, VK, RG, SP, NS, DR>::NT; \
    return true;                                        \
  }
  PKV_DL_VARIANTS(PKV_DT)
#undef PKV_DT
  return false;
}

hipError_t launch_dl(int lq, int lv, bool v_in_k, const AttnArgs& a, int64_t grid, hipStream_t s) {
#define PKV_DLL(Q, V, N, VK, RG, SP, NS, DR, M) \
  if (PKV_DL_MATCH(Q, V, VK, DR)) return launch_dl_t<Q, V, N, VK, RG, SP, NS, DR, M>(a, grid, s);
  PKV_DL_VARIANTS(PKV_DLL)
#undef PKV_DLL
  return hipErrorInvalidValue;
}

int dl_blocks_per_cu(int lq, int lv, bool v_in_k) {
#define PKV_DLO(Q, V, N, VK, RG, SP, NS, DR, M) \
  if (PKV_DL_MATCH(Q, V, VK, DR)) return dl_occupancy_t<Q, V, N, VK, RG, SP, NS, DR, M>();
  PKV_DL_VARIANTS(PKV_DLO)
#undef PKV_DLO
  return 1;
}

}  // namespace pkv
