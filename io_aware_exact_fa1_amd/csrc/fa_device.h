// Device helpers shared by the forward and backward kernels (gfx950).
// Internal header of the HIP library; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// XOR swizzle of the 16-byte chunk index within a K/V row: chunk c of row r
// is stored at chunk position c ^ swz(r).  Chosen for the two LDS read
// patterns of the kernel, with 64 banks of 4 bytes (256 bytes per cycle):
//  * K operand (ds_read_b128): 16 lanes read one chunk of 16 consecutive rows;
//  * V operand (ds_read_b64_tr_b16): 32 lanes read 4 consecutive chunks of
//    4 consecutive rows.
// d = 128 (one row = 256 bytes = all banks): the 16 rows need 16 distinct
// positions, and the 4 rows need distinct values in bits 2-3.  d = 64 (two
// rows per 256 bytes): rows of equal parity need 8 distinct positions, and
// rows r, r+2 of a 4-row group must differ in bit 2.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Symmetric reductions across the two 32-lane halves (lane l and l ^ 32):
// v_permlane32_swap(x, x) yields {x[l % 32], x[l % 32 + 32]} in every lane.
__device__ __forceinline__ float half_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Global -> LDS copies (global_load_lds_dwordx4): lane i writes LDS bytes
// [m0 + 16 i, m0 + 16 i + 16).  Issued through inline assembly so that the
// compiler does not make every later LDS read wait for them; the kernel
// waits for its copies itself (wait_copies) before the barrier that
// publishes them.  M0 is saved and restored around each copy.
//  lds_copy16: per-lane 64-bit source address.
//  lds_copy16_s: wave-uniform 64-bit base (SGPRs) + per-lane 32-bit offset.
__device__ __forceinline__ void lds_copy16(const void* src, unsigned lds_dst) {
  const unsigned base = __builtin_amdgcn_readfirstlane(lds_dst);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}
__device__ __forceinline__ void lds_copy16_s(const void* sbase, unsigned voff, unsigned lds_dst) {
  const unsigned base = __builtin_amdgcn_readfirstlane(lds_dst);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(base)
      : "memory");
}

// s_waitcnt vmcnt(n): at most n vector-memory operations of this wave still
// outstanding (they complete in order, so every older one has finished).
template <int n>
__device__ __forceinline__ void wait_copies() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (0xF << 8));
}

// Workgroup barrier that does not wait for outstanding global -> LDS copies
// (those are waited for explicitly): LDS accesses of this wave are complete
// and no memory access moves across it.  The scheduling barriers keep every
// instruction on its side, so the phases of the kernel loop stay as written.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Keep the computation of x on this side of the next phase barrier (the
// compiler would otherwise sink it to its first use in a later phase).
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void pin(bf16x8 x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void pin(f32x16 x) { asm volatile("" ::"v"(x)); }

}  // namespace fa
