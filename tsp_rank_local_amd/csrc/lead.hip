// Attention of rank 0's leading rows among themselves, in fp32. Positions
// below 64 see only keys below 64, all of them rank 0's own rows, so the
// layer recomputes those rows with fp32 intermediates; this is their
// attention step (exact expf softmax, fp32 products).
#include <math.h>

#include "device_common.h"
#include "tsp_internal.h"

namespace tsp {

// Attention of the first m <= 64 positions among themselves in fp32 (the
// leading rows of rank 0, whose keys are exactly those rows): one block per
// head, K and V of the m rows staged in LDS, four threads per query, each
// scoring 16 keys and later producing a quarter of the output features.
// q, o: [m][H][DH] fp32; k, v: [m][Hkv][DH] fp32, query head i reading K/V
// head i / (H / Hkv).
template <int DH>
__global__ __launch_bounds__(256) void lead_attn_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                        const float *__restrict__ v, float *__restrict__ o, int m,
                                                        int H, int Hkv, float scale) {
  __shared__ __attribute__((aligned(16))) float KP[64 * DH];  // K rows, later P [64][64]
  __shared__ __attribute__((aligned(16))) float Vs[64 * DH];
  const int head = blockIdx.x, tid = threadIdx.x;
  const int kvh = head / (H / Hkv);
  const int64_t rs = (int64_t)H * DH, kvs = (int64_t)Hkv * DH;
  for (int e = tid * 4; e < 64 * DH; e += 1024) {
    const int r = e / DH, d = e - r * DH;
    float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
    if (r < m) {
      kv = *reinterpret_cast<const float4 *>(k + r * kvs + kvh * DH + d);
      vv = *reinterpret_cast<const float4 *>(v + r * kvs + kvh * DH + d);
    }
    *reinterpret_cast<float4 *>(&KP[e]) = kv;
    *reinterpret_cast<float4 *>(&Vs[e]) = vv;
  }
  __syncthreads();
  const int i = tid >> 2, part = tid & 3;  // query i; keys (then features) of quarter part
  const float *qi = q + (int64_t)min(i, m - 1) * rs + head * DH;
  float sc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) sc[t] = 0.f;
  for (int d = 0; d < DH; d += 4) {
    const float4 qv = *reinterpret_cast<const float4 *>(qi + d);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float4 kv = *reinterpret_cast<const float4 *>(&KP[(16 * part + t) * DH + d]);
      sc[t] = fmaf(qv.x, kv.x, fmaf(qv.y, kv.y, fmaf(qv.z, kv.z, fmaf(qv.w, kv.w, sc[t]))));
    }
  }
  // causal: key j is visible to query i when j <= i
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 16; ++t)
    if (16 * part + t <= i) mx = fmaxf(mx, sc[t] * scale);
  mx = fmaxf(mx, __shfl_xor(mx, 1));
  mx = fmaxf(mx, __shfl_xor(mx, 2));
  float l = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    sc[t] = 16 * part + t <= i ? expf(sc[t] * scale - mx) : 0.f;
    l += sc[t];
  }
  l += __shfl_xor(l, 1);
  l += __shfl_xor(l, 2);
  __syncthreads();  // every score is taken: K's space now holds P
  const float inv = 1.0f / l;
#pragma unroll
  for (int t = 0; t < 16; ++t) KP[i * 64 + 16 * part + t] = sc[t] * inv;
  __syncthreads();
  constexpr int DQ = DH / 4;
  float acc[DQ];
#pragma unroll
  for (int dd = 0; dd < DQ; ++dd) acc[dd] = 0.f;
  for (int j = 0; j <= i; ++j) {
    const float pj = KP[i * 64 + j];
#pragma unroll
    for (int dd = 0; dd < DQ; dd += 4) {
      const float4 vv = *reinterpret_cast<const float4 *>(&Vs[j * DH + part * DQ + dd]);
      acc[dd] = fmaf(pj, vv.x, acc[dd]);
      acc[dd + 1] = fmaf(pj, vv.y, acc[dd + 1]);
      acc[dd + 2] = fmaf(pj, vv.z, acc[dd + 2]);
      acc[dd + 3] = fmaf(pj, vv.w, acc[dd + 3]);
    }
  }
  if (i < m) {
    float *oi = o + (int64_t)i * rs + head * DH + part * DQ;
#pragma unroll
    for (int dd = 0; dd < DQ; dd += 4)
      *reinterpret_cast<float4 *>(oi + dd) = make_float4(acc[dd], acc[dd + 1], acc[dd + 2], acc[dd + 3]);
  }
}

hipError_t launch_lead_attention(const float *q, const float *k, const float *v, float *o, int32_t m, int32_t H,
                                 int32_t Hkv, int32_t Dh, float scale, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  if (m > 64 || Hkv < 1 || H % Hkv != 0) return hipErrorInvalidValue;
  if (Dh == 128)
    hipLaunchKernelGGL((lead_attn_kernel<128>), dim3(H), dim3(256), 0, s, q, k, v, o, m, H, Hkv, scale);
  else
    hipLaunchKernelGGL((lead_attn_kernel<64>), dim3(H), dim3(256), 0, s, q, k, v, o, m, H, Hkv, scale);
  return hipGetLastError();
}

}  // namespace tsp
