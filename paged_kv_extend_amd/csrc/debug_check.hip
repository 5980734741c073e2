// Index validation of the debug build (libpkv_debug.so, compiled with
// PKV_DEBUG): before any attention kernel runs, the index and length arrays
// of a call are checked against the sizes the caller passed, so that an
// out-of-range pool slot or a malformed indptr becomes the error code
// PKV_ERR_RANGE instead of a wild read.  The release library compiles the
// kernel too but never launches it.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// flag bits: 1 qo_indptr, 2 kv_indptr, 4 a slot out of [0, pool_slots),
// 8 prefix_lens (negative)
__global__ __launch_bounds__(kThreads) void check_indices_kernel(CheckArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * kThreads;
  int bad = 0;
  for (int64_t b = tid; b < a.bs; b += nthreads) {
    if (a.qo_indptr) {
      if (a.qo_indptr[b + 1] < a.qo_indptr[b]) bad |= 1;
      if (b == 0 && a.qo_indptr[0] != 0) bad |= 1;
      if (b == a.bs - 1 && a.qo_indptr[a.bs] > a.total_q_tokens) bad |= 1;
    }
    if (a.kv_indptr[b + 1] < a.kv_indptr[b]) bad |= 2;
    if (b == 0 && a.kv_indptr[0] < 0) bad |= 2;
    if (b == a.bs - 1 && (int64_t)a.kv_indptr[a.bs] - a.kv_indptr[0] > a.num_indices) bad |= 2;
    if (a.prefix_lens && a.prefix_lens[b] < 0) bad |= 8;
  }
  if (bad) atomicOr(a.flag, bad);
  // (read only when the indptr checks above hold; a malformed indptr has
  // set the flag and the slots are not looked at)
  if (a.bs <= 0) return;
  const int64_t i0 = a.kv_indptr[0], i1 = a.kv_indptr[a.bs];
  if (i0 < 0 || i1 < i0 || i1 - i0 > a.num_indices) return;
  bad = 0;
  for (int64_t k = i0 + tid; k < i1; k += nthreads) {
    const int64_t s = a.kv_indices[k];
    if (s < 0 || s >= a.pool_slots) bad |= 4;
  }
  if (bad) atomicOr(a.flag, bad);
}

}  // namespace

hipError_t launch_check_indices(const CheckArgs& a, hipStream_t s) {
  const int64_t n = a.num_indices > a.bs ? a.num_indices : a.bs;
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(check_indices_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
