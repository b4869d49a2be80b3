// Internal helpers shared by the TokenGate HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "../../include/tokengate.h"

namespace tg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (NaN kept quiet).  The hardware
// conversion v_cvt_pk_bf16_f32 rounds the same way; this form is used where a
// single value is converted.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bf16x2 (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

// Order-preserving map of a float32 score to a uint32 key: larger score <=> larger
// key.  -0 and +0 share one key; every NaN maps to 0, below -inf (key 0x007fffff).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Cross-half exchange of a wave64: returns the value held by lane (lane ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// max / sum of the values held by lanes l and l^32, in every lane.  v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its second, so
// with both operands = x each lane ends up holding {x[l], x[l^32]} (in some order).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS byte address of a __shared__ object
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)(lds_void_t*)p;
}

// One 1 KiB global -> LDS DMA (global_load_lds_dwordx4): lane L reads 16 bytes at
// base + off and writes them at LDS byte m0v + 16 L.  base is a 64-bit scalar (wave-
// uniform) pointer, off a 32-bit per-lane byte offset, m0v the wave-uniform LDS
// destination; M0 is saved and restored around the issue.  Issued from inline asm so
// that the compiler does not make later LDS reads wait for it: the caller waits with
// s_waitcnt vmcnt and publishes the data with a barrier.
__device__ __forceinline__ void dma_lds16(uint32_t off, const void* base, uint32_t m0v) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "s"(m0v), "v"(off), "s"(base) : "memory");
}

// The same with the non-temporal cache policy, for data read exactly once.
__device__ __forceinline__ void dma_lds16_nt(uint32_t off, const void* base, uint32_t m0v) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3 nt\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "s"(m0v), "v"(off), "s"(base) : "memory");
}

// The same for 4 bytes per lane (global_load_lds_dword): LDS byte m0v + 4 L.
__device__ __forceinline__ void dma_lds4(uint32_t off, const void* base, uint32_t m0v) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "s"(m0v), "v"(off), "s"(base) : "memory");
}

// Wait until every DMA (and any other vector memory access) this wave issued has landed.
__device__ __forceinline__ void dma_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

#ifdef TG_DEBUG
// Debug builds: counts the violations of "pos strictly increasing and non-negative" on the
// stream, synchronises it, and returns TG_ERR_INVALID_ARG if there is any (tg_check.hip).
tg_status debug_check_positions(const int32_t* pos, int64_t m, void* stream);
#endif

}  // namespace tg

#define TG_CHECK_LAUNCH()                                   \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return TG_ERR_HIP; \
  } while (0)
