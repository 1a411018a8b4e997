// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace common {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr float kLn2 = 0.693147180559945309f;

// lanes l and l^32 hold the two key halves of the same query
__device__ __forceinline__ float max_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Workgroup barrier that is also a compiler barrier for memory operations but
// waits for nothing by itself: global->LDS copies in flight stay in flight
// across it.  Whatever must have landed before it is waited for explicitly by
// the caller (s_waitcnt), and every LDS read a wave issues is consumed, hence
// complete, before the barrier that follows it.
__device__ __forceinline__ void phase_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; a counter left at its maximum is not waited for).
template <int N>
constexpr int waitcnt_vm() {  // at most N vector-memory loads outstanding
  static_assert(N >= 0 && N < 64, "vmcnt range");
  return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);  // all LDS operations complete

// XOR key of a row's 16-byte chunks for rows of `chunks` chunks (a power of
// two).  With 16 chunks per row (d = 128) the 16 rows of one 16-lane group of
// a 128-bit K read get 16 different keys, and the 4 rows x 4 chunks of one
// 32-lane transposed V read land in 16 different chunk columns, so neither
// read has bank conflicts on the 64-bank LDS.
template <int CHUNKS>
__device__ __forceinline__ int swz(int row) {
  return (((row & 3) << 2) | ((row >> 2) & 3)) & (CHUNKS - 1);
}

// Start one 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4): lane
// l's 16 bytes land at lds_dst + 16*l (lds_dst is wave-uniform).  Issued from
// inline assembly so that the compiler does not track it: it would otherwise
// drain every copy in flight before each transposed LDS read it cannot prove
// disjoint.  Callers keep the ordering explicitly (s_waitcnt vmcnt before the
// barrier that publishes a slot; slots refilled only after their last reader).
// M0 carries the LDS destination and is set right before the copy; nothing
// else in these kernels uses M0 (a CPU test checks the generated code).
__device__ __forceinline__ void copy16_to_lds(const void* src, char* lds_dst) {
  const unsigned dst = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds_dst;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved; see the comment above
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(dst), "v"(src) : "m0");
#pragma clang diagnostic pop
}

// max(a, b, c) in one v_max3_f32 (the compiler forms it only sometimes).
// Inputs are finite or -inf, never NaN.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The same copy from base + voff: a wave-uniform 64-bit base (SGPRs) and a
// 32-bit per-lane byte offset, so a lane keeps one VGPR per copy instead of a
// 64-bit address.
__device__ __forceinline__ void copy16_to_lds(const void* base, unsigned voff, char* lds_dst) {
  const unsigned dst = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds_dst;
  // the base is wave-uniform by contract; readfirstlane states it to the
  // compiler, so that it is in SGPRs whatever the compiler proved about it
  const uint64_t b = (uint64_t)(uintptr_t)base;
  // (readfirstlane yields an int: widen through unsigned, never sign-extend)
  const uint64_t sb = ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32)) << 32) |
                      (uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)b);
  base = (const void*)(uintptr_t)sb;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved; see the comment above
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(dst), "v"(voff), "s"(base) : "m0");
#pragma clang diagnostic pop
}

// Two such copies 4096 bytes apart, from one offset register: base + voff_hi -
// 4096 -> lds_dst_hi - 4096, then base + voff_hi -> lds_dst_hi.  The
// instruction's immediate offset moves the global and the LDS address alike,
// so the pair needs one M0 write and one offset register (the immediate is a
// signed 13-bit field: -4096 fits, +4096 would not).  voff_hi >= 4096.
__device__ __forceinline__ void copy16x2_to_lds(const void* base, unsigned voff_hi, char* lds_dst_hi) {
  const unsigned dst = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds_dst_hi;
  const uint64_t b = (uint64_t)(uintptr_t)base;
  // (readfirstlane yields an int: widen through unsigned, never sign-extend)
  const uint64_t sb = ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32)) << 32) |
                      (uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)b);
  base = (const void*)(uintptr_t)sb;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved; see copy16_to_lds
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:-4096\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(dst), "v"(voff_hi), "s"(base)
      : "m0");
#pragma clang diagnostic pop
}

}  // namespace common
}  // namespace fa
