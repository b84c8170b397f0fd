// Causal attention of one rank's zigzag-ordered queries against the gathered
// full-sequence K/V, on the gfx950 matrix cores.
//
// Work split: the rank's local rows form two chunks (global positions r*C..
// and (2D-1-r)*C..). They are cut into T = ceil(C/128) query tiles per chunk;
// block (head, p) takes tile p of the first chunk and the mirrored tile
// T-1-p of the second, so every block walks about S/64 + 2 key tiles and all
// blocks carry equal causal work. Key tiles past a tile's last query are never
// loaded; only tiles that straddle the diagonal apply the mask.
//
// Per block: 4 waves x 32 queries. Per 64-key tile the block stages K (bf16,
// row-major, 16-byte chunks XOR-swizzled by row) and V (converted to fp16 and
// stored transposed, 8-byte units XOR-swizzled by feature) in LDS, two stages
// deep, with the next tile's global loads issued before the current tile's
// math. Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so a
// lane owns one query and 32 of the tile's keys: the row max needs one
// exchange between the two half-waves, and the row sum none until the end.
// Softmax runs in the exp2 domain with the scale folded into one FMA; the
// probabilities are rounded to fp16 (v_cvt_pk_f16_f32) and summed from those
// rounded values (v_dot2c_f32_f16), and O^T = V^T P^T runs on
// v_mfma_f32_32x32x16_f16 with P taken straight from the score registers. The
// O rescale is skipped when no query of the wave raised its running max.
//
// A plain fp32 kernel (one thread per query, exact expf) serves fp32 inputs.
#include <math.h>

#include "device_common.h"
#include "tsp_internal.h"

namespace tsp {

struct AttnArgs {
  const void *q, *k, *v;
  void *o;
  int64_t S;
  int32_t n, H;
  float scale;  // softmax scale
  float c;      // scale * log2(e)
  ZigzagMap zz;
  int32_t T;  // query tiles per chunk
};

constexpr int kBQ = 128, kBKey = 64, kAttnThreads = 256;

template <int DH>
__device__ __forceinline__ int k_swz(int row, int ch) {  // element offset of chunk ch of K row
  constexpr int CPR = DH / 8;
  const int f = CPR == 16 ? (row & 15) : ((row >> 1) & 7);
  return row * DH + ((ch ^ f) << 3);
}
__device__ __forceinline__ int v_swz(int d, int unit) {  // element offset of 4-key unit of V^T row d
  return d * kBKey + ((unit ^ ((d >> 1) & 15)) << 2);
}

template <int DH, bool OUT_F32>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int CPR = DH / 8;                 // 16-byte chunks per K row
  constexpr int K_LD = (kBKey * CPR) / kAttnThreads;  // K chunks per thread
  constexpr int V_UNITS = 16 * (DH / 8);      // (4 keys x 8 features) units per tile
  constexpr int ND = DH / 32;                 // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][kBKey * DH];
  __shared__ __attribute__((aligned(16))) _Float16 Vt[2][DH * kBKey];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head = L / a.T, p = L - (L / a.T) * a.T;
  const int64_t rs = (int64_t)a.H * DH;  // row pitch of q, k, v, o
  const bf16 *qg = reinterpret_cast<const bf16 *>(a.q) + head * DH;
  const bf16 *kg = reinterpret_cast<const bf16 *>(a.k) + head * DH;
  const bf16 *vg = reinterpret_cast<const bf16 *>(a.v) + head * DH;

  u32x4 rk[K_LD], rv[4];
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBKey;
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int c = tid + kAttnThreads * i;
      const int row = c / CPR, ch = c % CPR;
      const int64_t key = k0 + row;
      u32x4 zero = {0u, 0u, 0u, 0u};
      rk[i] = key < a.S ? *reinterpret_cast<const u32x4 *>(kg + key * rs + ch * 8) : zero;
    }
    if (tid < V_UNITS) {
      const int doct = tid % (DH / 8), kq = tid / (DH / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t key = k0 + kq * 4 + i;
        u32x4 zero = {0u, 0u, 0u, 0u};
        rv[i] = key < a.S ? *reinterpret_cast<const u32x4 *>(vg + key * rs + doct * 8) : zero;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int c = tid + kAttnThreads * i;
      const int row = c / CPR, ch = c % CPR;
      *reinterpret_cast<u32x4 *>(&Ks[buf][k_swz<DH>(row, ch)]) = rk[i];
    }
    if (tid < V_UNITS) {
      const int doct = tid % (DH / 8), kq = tid / (DH / 8);
      bf16x8 vb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vb[i] = __builtin_bit_cast(bf16x8, rv[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f16x4 u;
        u[0] = (_Float16)(float)vb[0][e];
        u[1] = (_Float16)(float)vb[1][e];
        u[2] = (_Float16)(float)vb[2][e];
        u[3] = (_Float16)(float)vb[3][e];
        *reinterpret_cast<f16x4 *>(&Vt[buf][v_swz(doct * 8 + e, kq)]) = u;
      }
    }
  };

  for (int half = 0; half < 2; ++half) {
    const int tile = half == 0 ? p : 2 * a.T - 1 - p;
    const int ch_half = tile < a.T ? 0 : 1;
    const int row0 = ch_half * a.zz.C + (tile - ch_half * a.T) * kBQ;  // first local row of the tile
    const int nvalid = min(kBQ, (ch_half + 1) * a.zz.C - row0);
    const int pos0 = a.zz.pos(row0);  // positions are consecutive inside a tile
    const int n_kt = (pos0 + nvalid - 1) / kBKey + 1;

    const int wrow0 = wave * 32;
    const int w_nvalid = max(0, min(32, nvalid - wrow0));
    const int wmin = pos0 + wrow0, wmax = pos0 + wrow0 + w_nvalid - 1;
    const bool my_valid = wrow0 + l32 < nvalid;
    const int qpos = pos0 + min(wrow0 + l32, nvalid - 1);
    const int64_t qrow = row0 + wrow0 + l32;

    bf16x8 qf[DH / 16];
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk) {
      if (my_valid) {
        qf[kk] = *reinterpret_cast<const bf16x8 *>(qg + qrow * rs + kk * 16 + g * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[kk][e] = (bf16)0.f;
      }
    }

    f32x16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m_run = -INFINITY, l_part = 0.f;

    gload(0);
    sstore(0);
    __syncthreads();

    for (int kt = 0; kt < n_kt; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < n_kt) gload(kt + 1);
      const int kstart = kt * kBKey;
      if (w_nvalid > 0 && kstart <= wmax) {
        // ---- S^T = K Q^T for the 64 keys of this tile
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
          for (int kk = 0; kk < DH / 16; ++kk) {
            const int row = kb * 32 + l32;
            const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&Ks[cur][k_swz<DH>(row, kk * 2 + g)]);
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[kb], 0, 0, 0);
          }
        }
        // sacc[kb][v] is the score of key kstart + kb*32 + 8*(v/4) + 4*g + v%4
        const bool need_mask = kstart + kBKey - 1 > wmin;
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int key = kstart + kb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
              if (key > qpos) sacc[kb][v] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
        mx = halves_max(mx);
        const float mxs = mx == -INFINITY ? -INFINITY : mx * a.c;
        const float m_new = fmaxf(m_run, mxs);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        // ---- probabilities (fp16) and their partial row sum
        f16x8 pf[2][2];
        float psum = 0.f;
        const _Float16 one = (_Float16)1.0f;
        const f16x2 ones = {one, one};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][hh * 8 + e], a.c, -m_new));
              float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][hh * 8 + e + 1], a.c, -m_new));
              if (need_mask) {
                const int key0 = kstart + kb * 32 + (hh * 2 + (e >> 2)) * 8 + g * 4 + (e & 3);
                if (key0 > qpos) p0 = 0.f;
                if (key0 + 1 > qpos) p1 = 0.f;
              }
              f16x2 pr = {(_Float16)p0, (_Float16)p1};
              pf[kb][hh][e] = pr[0];
              pf[kb][hh][e + 1] = pr[1];
              psum = __builtin_amdgcn_fdot2(pr, ones, psum, false);
            }
        l_part = l_part * alpha + psum;
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
        }
        // ---- O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            const int d = db * 32 + l32;
            const f16x4 lo = *reinterpret_cast<const f16x4 *>(&Vt[cur][v_swz(d, kq * 4 + g)]);
            const f16x4 hi = *reinterpret_cast<const f16x4 *>(&Vt[cur][v_swz(d, kq * 4 + 2 + g)]);
            const f16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[kq >> 1][kq & 1], oacc[db], 0, 0, 0);
          }
        }
      }
      if (kt + 1 < n_kt) sstore(cur ^ 1);
      __syncthreads();
    }

    // ---- normalise and store: oacc[db][v] is O[query][db*32 + 8*(v/4) + 4*g + v%4]
    const float inv = 1.0f / halves_sum(l_part);
    if (my_valid) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const int d0 = db * 32 + vq * 8 + g * 4;
          const float o0 = oacc[db][vq * 4 + 0] * inv, o1 = oacc[db][vq * 4 + 1] * inv;
          const float o2 = oacc[db][vq * 4 + 2] * inv, o3 = oacc[db][vq * 4 + 3] * inv;
          if constexpr (OUT_F32) {
            float *og = reinterpret_cast<float *>(a.o) + qrow * rs + head * DH + d0;
            *reinterpret_cast<float4 *>(og) = make_float4(o0, o1, o2, o3);
          } else {
            bf16 *og = reinterpret_cast<bf16 *>(a.o) + qrow * rs + head * DH + d0;
            og[0] = (bf16)o0;
            og[1] = (bf16)o1;
            og[2] = (bf16)o2;
            og[3] = (bf16)o3;
          }
        }
    }
  }
}

// fp32 inputs: one thread per query row, keys staged 64 at a time in LDS,
// exact per-key online softmax with expf.
template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ float Ks[64][DH + 1];
  __shared__ float Vs[64][DH];
  const int tid = threadIdx.x, head = blockIdx.y;
  const int row = blockIdx.x * 64 + tid;
  const bool valid = row < a.n;
  const int last_row = min(a.n - 1, (int)blockIdx.x * 64 + 63);
  const int max_pos = a.zz.pos(last_row);  // positions grow with the local row
  const int qpos = a.zz.pos(valid ? row : last_row);
  const int64_t rs = (int64_t)a.H * DH;
  const float *q = reinterpret_cast<const float *>(a.q) + head * DH;
  const float *k = reinterpret_cast<const float *>(a.k) + head * DH;
  const float *v = reinterpret_cast<const float *>(a.v) + head * DH;
  float qv[DH], ov[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    qv[d] = valid ? q[(int64_t)row * rs + d] : 0.f;
    ov[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 <= max_pos; k0 += 64) {
    const int64_t key = k0 + tid;
    for (int d = 0; d < DH; ++d) {
      Ks[tid][d] = key < a.S ? k[key * rs + d] : 0.f;
      Vs[tid][d] = key < a.S ? v[key * rs + d] : 0.f;
    }
    __syncthreads();
    const int nk = min(64, qpos - k0 + 1);
    for (int u = 0; u < nk; ++u) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) s = fmaf(qv[d], Ks[u][d], s);
      s *= a.scale;
      const float m_new = fmaxf(m, s);
      const float alpha = expf(m - m_new);
      const float pr = expf(s - m_new);
      l = l * alpha + pr;
#pragma unroll
      for (int d = 0; d < DH; ++d) ov[d] = fmaf(pr, Vs[u][d], ov[d] * alpha);
      m = m_new;
    }
    __syncthreads();
  }
  if (valid) {
    float *o = reinterpret_cast<float *>(a.o) + (int64_t)row * rs + head * DH;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < DH; ++d) o[d] = ov[d] * inv;
  }
}

hipError_t launch_attention(int dtype, const void *q, const void *k, const void *v, void *o, int o_dtype,
                            int64_t S, int32_t n, int32_t H, int32_t Dh, float scale, ZigzagMap zz,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.S = S;
  a.n = n;
  a.H = H;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  a.zz = zz;
  a.T = (zz.C + kBQ - 1) / kBQ;
  if (dtype == TSP_BF16) {
    dim3 grid(H * a.T);
    const bool f32out = o_dtype == TSP_F32;
    if (Dh == 128) {
      if (f32out)
        hipLaunchKernelGGL((attn_bf16_kernel<128, true>), grid, dim3(kAttnThreads), 0, s, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<128, false>), grid, dim3(kAttnThreads), 0, s, a);
    } else {
      if (f32out)
        hipLaunchKernelGGL((attn_bf16_kernel<64, true>), grid, dim3(kAttnThreads), 0, s, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<64, false>), grid, dim3(kAttnThreads), 0, s, a);
    }
  } else {
    dim3 grid((n + 63) / 64, H);
    if (Dh == 128)
      hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace tsp
