// Merge of the chunks of a split item, fused into the attention kernels: the
// workgroup that writes the last chunk's partial state combines all of them.
//
// In chunk order (deterministic, whichever chunk finishes last):
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o = sum_s acc_s 2^(m_s - M) / L
// the log-sum-exp state merge (page "flashinfer_backend.py", forward_extend:
// merge_state of the ragged and paged partial outputs).
#pragma once

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

// Rows of split item mi from its partial states into o; thread = (row, 4 columns).
template <bool F32, int LV>
__device__ void merge_tile(const AttnArgs& a, const MergeItem& mi, int bm, int tid, int nthreads) {
  const int G = a.group;
  const int q0 = a.qo_indptr[mi.b], E = a.qo_indptr[mi.b + 1] - q0;
  const int R = E * G;
  constexpr int V4 = LV / 4;
  for (int idx = tid; idx < bm * V4; idx += nthreads) {
    const int row = idx / V4, d = (idx % V4) * 4;
    const int r = mi.t * bm + row;
    if (r >= R) continue;
    float M = -INFINITY;
    for (int s = 0; s < mi.n; ++s) M = fmaxf(M, a.part_ml[((int64_t)(mi.part_base + s) * bm + row) * 2]);
    float L = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < mi.n; ++s) {
      const int64_t prow = (int64_t)(mi.part_base + s) * bm + row;
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + prow * 2);
      const float w = ml.x == -INFINITY ? 0.0f : fast_exp2(ml.x - M);
      L += ml.y * w;
      const float4 v = *reinterpret_cast<const float4*>(a.part_acc + prow * LV + d);
      o.x += v.x * w;
      o.y += v.y * w;
      o.z += v.z * w;
      o.w += v.w * w;
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

// Called by every thread of a workgroup after it wrote the partial state of
// one chunk of split item a.merge[merge_index]: the chunks count themselves
// in, and the workgroup that brings the count to n merges them.  Release:
// each workgroup's partial writes are visible device-wide before its count;
// acquire: the last one reads the others' after seeing the full count.
template <bool F32, int LV>
__device__ void finish_split(const AttnArgs& a, int merge_index, int bm) {
  __shared__ int last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int n = a.merge[merge_index].n;
    last = atomicAdd(&a.merge[merge_index].arrived, 1) == n - 1;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  merge_tile<F32, LV>(a, a.merge[merge_index], bm, threadIdx.x, blockDim.x);
}

}  // namespace pkv
