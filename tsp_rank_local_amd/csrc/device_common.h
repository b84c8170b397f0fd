// Device-side helpers shared by the gfx950 kernels: vector types for MFMA
// operands, bf16/fp16 conversions and wave-level exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// s_waitcnt immediate that waits for every outstanding vector-memory load
// (vmcnt = 0) and leaves the export and LDS/scalar counters unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16 b) { return (float)b; }
// Round to nearest even (gfx950 converts with v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16 f32_to_bf16(float f) { return (bf16)f; }

// Exact GELU z * Phi(z) in fp32.
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// For a value held by every lane, combine it with the value of lane l^32.
// v_permlane32_swap exchanges the upper half of one register with the lower
// half of another; fed the same value twice, the two results hold, in every
// lane, the values of lane l and lane l^32 (in some order), so symmetric
// combines need not know which is which.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Blocks are handed to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Remap so that consecutive logical tiles land on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  if ((nblocks & 7) != 0) return b;
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

}  // namespace tsp
