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

// GELU z * Phi(z) = z * (1 + erf(z / sqrt 2)) / 2 in fp32, with erf from the
// rational approximation of Abramowitz and Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: for x >= 0, erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3
// + a4 t^4 + a5 t^5) exp(-x^2) + e(x), t = 1 / (1 + p x), |e(x)| <= 1.5e-7.
// With q = (1 - erf(|z|/sqrt 2)) / 2, GELU(z) = z (1 - q) for z >= 0 and
// z q for z < 0 (erf is odd). About 17 VALU ops against ~40 for erff.
__device__ __forceinline__ float gelu_erf(float z) {
  constexpr float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
                  a4 = -1.453152027f, a5 = 1.061405429f;
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, x, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  // exp(-x^2) = exp2(-z^2 / 2 * log2(e))
  const float e = __builtin_amdgcn_exp2f(z * z * -0.72134752044448170f);
  const float q = 0.5f * poly * e;
  return z * (z >= 0.0f ? 1.0f - q : q);
}

// GELU'(z) = Phi(z) + z phi(z) in fp32, phi(z) = exp(-z^2/2) / sqrt(2 pi):
// Phi from the same erf approximation as gelu_erf, and exp(-z^2/2) is the
// factor that approximation already needs.
__device__ __forceinline__ float gelu_erf_grad(float z) {
  constexpr float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
                  a4 = -1.453152027f, a5 = 1.061405429f;
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, x, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  const float e = __builtin_amdgcn_exp2f(z * z * -0.72134752044448170f);
  const float q = 0.5f * poly * e;
  return fmaf(z * 0.39894228040143268f, e, z >= 0.0f ? 1.0f - q : q);
}

// SiLU z * sigma(z) = z / (1 + e^-z) in fp32, e^-z as exp2(-z log2 e): for
// z -> -inf, e^-z overflows to inf and the result goes to -0; for z -> +inf
// it goes to z.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
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

#if defined(__HIP_DEVICE_COMPILE__)
// ---------------------------------------------------------------- HBM -> LDS copies
// Wait until at most N vector-memory operations of this wave are outstanding
// (N < 64; the count's low 4 bits sit in bits 3:0 of the s_waitcnt immediate
// and its high 2 bits in bits 15:14; export and LDS/scalar counters are left
// unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Raw buffer descriptor over [base, base + bytes): base, base high with stride
// 0, size in bytes, raw-buffer format. Loads at offsets >= bytes return zeros.
__device__ __forceinline__ u32x4 buffer_rsrc(const void *base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = (uint32_t)b;
  r[1] = (uint32_t)(b >> 32) & 0xFFFFu;
  r[2] = bytes;
  r[3] = 0x00020000u;
  return r;
}

// LDS byte address of a __shared__ object (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)(p));
}

// One 16-byte-per-lane copy from a buffer straight into LDS: lane i's 16
// bytes at voffset + soffset land at lds_base + 16*i (buffer_load ... lds).
// Issued as plain asm so that the compiler does not treat every later LDS
// read as a possible reader of this copy (it would then wait for all copies
// in flight, from HBM, before each read); callers order every copy before
// its readers themselves (vmcnt waits and block barriers).
// M0 holds the LDS address of the copy. The compiler reserves M0 and notes
// the clobber only as a warning, so these helpers set it on every use and are
// used only in kernels with no other M0 user (no LDS-DMA builtins there).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(u32x4 rsrc, int voffset, int soffset, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"  // one wait state between an M0 write and an LDS copy
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "s"(soffset), "s"(lds_base)
      : "memory", "m0");
}

// Same with 4 bytes per lane (lane i -> lds_base + 4*i). Used to pull lines
// into L2 ahead of their copies: the data lands in a scratch LDS area nobody
// reads, so no register has to stay reserved while the load is in flight.
__device__ __forceinline__ void lds_touch4(u32x4 rsrc, int voffset, int soffset, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, %2 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "s"(soffset), "s"(lds_base)
      : "memory", "m0");
}
#pragma clang diagnostic pop
#endif  // __HIP_DEVICE_COMPILE__

// Blocks are handed to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Remap so that consecutive logical tiles land on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  if ((nblocks & 7) != 0) return b;
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

}  // namespace tsp
