// Shared device/host helpers of the HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bsa.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *(u32x4 *)p = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ unsigned bf16_bits(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
  return __builtin_bit_cast(float, (unsigned)b << 16);
}

// Swap with the lane 32 apart (the other half of a 64-lane wave).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

inline int status_of(hipError_t e) { return e == hipSuccess ? BSA_OK : BSA_ERR_HIP; }

// hipGetLastError also returns an error that an earlier, unrelated HIP call
// of the same thread left pending (a runtime probe of the caller's framework,
// say).  Every launcher clears that first, so that the status it returns
// after its launches speaks of its own launches only.
inline void clear_pending_error() { (void)hipGetLastError(); }

}  // namespace bsa
