// Device helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// global (address space 1) and LDS (address space 3) pointers
template <class T>
using gptr = const __attribute__((address_space(1))) T*;
template <class T>
using lptr = __attribute__((address_space(3))) T*;

constexpr float kLog2e = 1.4426950408889634f;
// base-2 headroom before the reference max of the online softmax is raised
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value over lanes l and l ^ 32
__device__ __forceinline__ float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt encodings (gfx9: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
// Each wait is also a compiler memory fence: the loads it guards (LDS data
// written by global-to-LDS loads the compiler does not track) stay after it.
// vmcnt(0) lgkmcnt(0)
__device__ __forceinline__ void wait_all_mem() {
  __builtin_amdgcn_s_waitcnt(0x7 << 4);
  asm volatile("" ::: "memory");
}
// lgkmcnt(0) only: LDS traffic done, global loads may stay in flight
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}
// vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
  asm volatile("" ::: "memory");
}

// Workgroup barrier that is also a compiler memory fence (no LDS access is
// moved across it).  The waits that must precede it are the caller's.
__device__ __forceinline__ void barrier_fence() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4; the wave-uniform LDS base goes through M0).
// Issued from inline assembly so that the compiler does not track an LDS
// write in flight: it would otherwise wait for every such load before each
// transposing LDS read, serialising the next tile's loads with this tile's
// math.  Kernels wait for these loads themselves (vmcnt) before the barrier
// that publishes a tile, and must not read the destination before that.
// M0 is saved and restored around the load (the compiler reserves it), with
// one wait state between each write of M0 and the load.  No memory clobber:
// the asm is volatile, so it keeps its order against the fenced waits and
// barriers that bound every use of its destination, and the compiler stays
// free to schedule the LDS operand reads of other stages around it.
__device__ __forceinline__ void load_lds_16(gptr<void> src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base));
}

// 4 bytes per active lane from global memory into LDS at lds_base + 4 * lane
// (global_load_lds_dword); same conventions as load_lds_16.
__device__ __forceinline__ void load_lds_4(gptr<void> src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lptr<const void>)p; }

// A wave-uniform 64-bit value pinned to scalar registers (the compiler cannot
// turn its later uses back into memory loads).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace pkv
