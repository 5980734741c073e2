// Merge of the chunks of split items, a launch of its own after the attention
// launch.  In chunk order (deterministic), batch by batch:
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o = sum_s acc_s 2^(m_s - M) / L
// the log-sum-exp state merge (page "flashinfer_backend.py", forward_extend:
// merge_state of the ragged and paged partial outputs), plus the sink term.
//
// The attention launch only writes each chunk's partial state: on MI355X each
// XCD has an L2 of its own, so a chunk that published its state to a merging
// workgroup on another XCD inside the launch would need a device-scope
// release (an L2 write-back) per chunk; the launch boundary orders the writes
// for free.  A chunk's workgroup is then done as soon as its writes are
// issued, and the merges run spread over every CU.
#pragma once

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kMergeBatch = 16;  // partial states loaded together per thread

// Work of the merge launch: (merge record, block of rows) tasks, strided over
// the grid; thread = (row of the block, 4 columns).  Rows hold lv columns
// (partial accumulators are lv floats apart); LVP, a power of two >= lv,
// sets the threads per row, and threads past lv idle.
template <bool F32, int LVP>
__global__ __launch_bounds__(256) void split_merge_kernel(AttnArgs a, int bm, int lv) {
  constexpr int V4 = LVP / 4;         // float4 columns per row
  constexpr int RPB = 256 / V4;       // rows per task
  static_assert(256 % V4 == 0, "columns per thread block");
  const int blocks = (bm + RPB - 1) / RPB;
  const int tasks = a.hdr->num_merge * blocks;
  const int row_in = threadIdx.x / V4, d = 4 * (threadIdx.x % V4);
  const int G = a.group;
  for (int task = blockIdx.x; task < tasks; task += gridDim.x) {
    const MergeItem mi = a.merge[task / blocks];
    const int row = (task % blocks) * RPB + row_in;
    const int q0 = mi.q0, E = mi.E;
    const int r = mi.t * bm + row;
    if (row >= bm || r >= E * G || d >= lv) continue;
    // pieces in batches of kMergeBatch, every load of a batch in flight at
    // once; the running state is rescaled when a batch raises the maximum
    float M = -INFINITY, L = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < mi.n; s0 += kMergeBatch) {
      float2 ml[kMergeBatch];
      float4 v[kMergeBatch];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        ml[i] = make_float2(-INFINITY, 0.0f);
        v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (s0 + i < mi.n) {
          const int64_t prow = (int64_t)(mi.part_base + s0 + i) * bm + row;
          ml[i] = *reinterpret_cast<const float2*>(a.part_ml + prow * 2);
          v[i] = *reinterpret_cast<const float4*>(a.part_acc + prow * lv + d);
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
        const float w = ml[i].x == -INFINITY ? 0.0f : fast_exp2(ml[i].x - M);
        L += ml[i].y * w;
        o.x += v[i].x * w;
        o.y += v[i].y * w;
        o.z += v[i].z * w;
        o.w += v[i].w * w;
      }
    }
    const int tok = r / G, head = mi.g * G + r % G;
    if (a.sinks) L += fast_exp2(a.sinks[head] * kLog2e - M);
    const float inv = 1.0f / L;
    const int64_t off = (int64_t)(q0 + tok) * a.o_st + (int64_t)head * a.o_sh + d;
    if constexpr (F32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + off) =
          make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    } else {
      bf16x4 ov;
      ov[0] = (__bf16)(o.x * inv);
      ov[1] = (__bf16)(o.y * inv);
      ov[2] = (__bf16)(o.z * inv);
      ov[3] = (__bf16)(o.w * inv);
      *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(a.o) + off) = ov;
    }
  }
}

}  // namespace pkv
