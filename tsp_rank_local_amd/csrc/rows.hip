// Row-wise kernels: zigzag index map and RMSNorm (fp32 in, bf16/fp32 out).
#include "device_common.h"
#include "tsp_internal.h"

namespace tsp {

__global__ void zigzag_index_kernel(ZigzagMap zz, int32_t n, int32_t *pos) {
  int32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) pos[t] = zz.pos(t);
}

hipError_t launch_zigzag_index(ZigzagMap zz, int32_t n, int32_t *pos, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int threads = 256;
  int blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(zigzag_index_kernel, dim3(blocks), dim3(threads), 0, s, zz, n, pos);
  return hipGetLastError();
}

// One 256-thread block per row; h % 4 == 0. The sum of squares runs in fp32,
// first per thread, then across the wave with shuffles, then across waves.
// panel_stride > 0: out in panel layout (64-column panels of [rows][64]).
// CACHED (h <= 8192): each thread keeps its float4 columns (4 * thread +
// 1024 * i) in registers between the sum and the output, so the row is read
// from memory once; otherwise it is read twice.
template <typename T>
__device__ __forceinline__ void put4(T *o, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4 *>(o) = make_float4(a, b, c, d);
  } else {
    const bf16x2 lo = {(bf16)a, (bf16)b}, hi = {(bf16)c, (bf16)d};
    *reinterpret_cast<u32x2 *>(o) = u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  }
}

constexpr int kNormChunks = 8;  // float4 columns per thread with CACHED

template <typename G, typename O, bool CACHED>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ x, const G *__restrict__ g,
                                                      O *__restrict__ out, int32_t h, float eps, int64_t panel_stride) {
  const int64_t row = blockIdx.x;
  const float *xr = x + row * h;
  float ss = 0.f;
  float4 xv[CACHED ? kNormChunks : 1];
  if constexpr (CACHED) {
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
      const int c = threadIdx.x * 4 + 1024 * i;
      xv[i] = c < h ? *reinterpret_cast<const float4 *>(xr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      ss += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
    }
  } else {
    for (int c = threadIdx.x * 4; c < h; c += 1024) {
      float4 v = *reinterpret_cast<const float4 *>(xr + c);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  __shared__ float part[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  float tot = part[0] + part[1] + part[2] + part[3];
  const float rstd = 1.0f / sqrtf(tot / (float)h + eps);
  auto emit = [&](int c, float4 v) {
    O *o = out + (panel_stride ? panel_index(row, c, panel_stride) : row * h + c);  // 4 elements, one panel
    put4(o, v.x * rstd * (float)g[c + 0], v.y * rstd * (float)g[c + 1], v.z * rstd * (float)g[c + 2],
         v.w * rstd * (float)g[c + 3]);
  };
  if constexpr (CACHED) {
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
      const int c = threadIdx.x * 4 + 1024 * i;
      if (c < h) emit(c, xv[i]);
    }
  } else {
    for (int c = threadIdx.x * 4; c < h; c += 1024) emit(c, *reinterpret_cast<const float4 *>(xr + c));
  }
}

template <typename G, typename O>
static void launch_rmsnorm_rows(const float *x, const G *g, O *out, int32_t rows, int32_t h, float eps, int64_t ps,
                                hipStream_t s) {
  if (h <= 1024 * kNormChunks)
    hipLaunchKernelGGL((rmsnorm_kernel<G, O, true>), dim3(rows), dim3(256), 0, s, x, g, out, h, eps, ps);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<G, O, false>), dim3(rows), dim3(256), 0, s, x, g, out, h, eps, ps);
}

hipError_t launch_rmsnorm(const float *x, const void *g, void *out, int32_t rows, int32_t h, float eps,
                          int dtype, bool out_panel, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t ps = out_panel ? (int64_t)rows * kPanel : 0;
  if (dtype == TSP_BF16)
    launch_rmsnorm_rows(x, (const bf16 *)g, (bf16 *)out, rows, h, eps, ps, s);
  else
    launch_rmsnorm_rows(x, (const float *)g, (float *)out, rows, h, eps, ps, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- RMSNorm backward
// Backward of rmsnorm_kernel. With r = (mean(x^2) + eps)^(-1/2) and output
// x_k g_k r, the gradient of row x for output gradient d is
//   dx_k = r g_k d_k - x_k r^3 / h * sum_i d_i g_i x_i,
// and the gain receives sum over rows of d_k x_k r. A block takes
// kNormBwdRows consecutive rows; each thread keeps its float4 columns
// (c = 4 * thread + 1024 * i) of x and d in registers between the two row
// sums and the output, and adds d x r into per-column partial sums that the
// block writes to part[block][h]. rmsnorm_bwd_dg_kernel adds those rows in
// block order, so the gain gradient does not depend on scheduling.
constexpr int kNormBwdRows = 16, kNormBwdChunks = 8;  // h <= 4 * 256 * 8

template <typename G, typename L>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float *__restrict__ x, const G *__restrict__ g,
                                                          const float *__restrict__ d, const float *__restrict__ res,
                                                          float *__restrict__ dx, L *__restrict__ lo, int64_t lo_panel,
                                                          int32_t rows, int32_t h, float eps,
                                                          float *__restrict__ part) {
  float4 gg[kNormBwdChunks], acc[kNormBwdChunks];
#pragma unroll
  for (int i = 0; i < kNormBwdChunks; ++i) {
    const int c = threadIdx.x * 4 + 1024 * i;
    gg[i] = c < h ? make_float4((float)g[c], (float)g[c + 1], (float)g[c + 2], (float)g[c + 3])
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __shared__ float2 red[2][4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int rr = 0; rr < kNormBwdRows; ++rr) {
    const int64_t row = (int64_t)blockIdx.x * kNormBwdRows + rr;
    if (row >= rows) break;  // the same for the whole block
    const float *xr = x + row * h, *dr = d + row * h;
    float4 xv[kNormBwdChunks], dv[kNormBwdChunks];
    float ss = 0.f, sdgx = 0.f;
#pragma unroll
    for (int i = 0; i < kNormBwdChunks; ++i) {
      const int c = threadIdx.x * 4 + 1024 * i;
      xv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      dv[i] = xv[i];
      if (c < h) {
        xv[i] = *reinterpret_cast<const float4 *>(xr + c);
        dv[i] = *reinterpret_cast<const float4 *>(dr + c);
      }
      ss += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
      sdgx += dv[i].x * gg[i].x * xv[i].x + dv[i].y * gg[i].y * xv[i].y + dv[i].z * gg[i].z * xv[i].z +
              dv[i].w * gg[i].w * xv[i].w;
    }
    for (int off = 32; off > 0; off >>= 1) {
      ss += __shfl_xor(ss, off);
      sdgx += __shfl_xor(sdgx, off);
    }
    // two slots: a wave that runs ahead into the next row writes the other
    // one, and cannot reach this slot again before every wave has passed
    // the next row's barrier (after its reads here)
    if (lane == 0) red[rr & 1][wave] = make_float2(ss, sdgx);
    __syncthreads();
    const float2 t0 = red[rr & 1][0], t1 = red[rr & 1][1], t2 = red[rr & 1][2], t3 = red[rr & 1][3];
    const float tss = t0.x + t1.x + t2.x + t3.x, tsd = t0.y + t1.y + t2.y + t3.y;
    const float r = 1.0f / sqrtf(tss / (float)h + eps);
    const float k = r * r * r * tsd / (float)h;
#pragma unroll
    for (int i = 0; i < kNormBwdChunks; ++i) {
      const int c = threadIdx.x * 4 + 1024 * i;
      if (c >= h) continue;
      float4 o = make_float4(r * gg[i].x * dv[i].x - k * xv[i].x, r * gg[i].y * dv[i].y - k * xv[i].y,
                             r * gg[i].z * dv[i].z - k * xv[i].z, r * gg[i].w * dv[i].w - k * xv[i].w);
      if (res) {
        const float4 a = *reinterpret_cast<const float4 *>(res + row * h + c);
        o = make_float4(o.x + a.x, o.y + a.y, o.z + a.z, o.w + a.w);
      }
      *reinterpret_cast<float4 *>(dx + row * h + c) = o;
      if (lo) {
        L *p = lo + (lo_panel ? panel_index(row, c, lo_panel) : row * h + c);  // 4 elements, one panel
        p[0] = (L)o.x;
        p[1] = (L)o.y;
        p[2] = (L)o.z;
        p[3] = (L)o.w;
      }
      acc[i].x += dv[i].x * xv[i].x * r;
      acc[i].y += dv[i].y * xv[i].y * r;
      acc[i].z += dv[i].z * xv[i].z * r;
      acc[i].w += dv[i].w * xv[i].w * r;
    }
  }
#pragma unroll
  for (int i = 0; i < kNormBwdChunks; ++i) {
    const int c = threadIdx.x * 4 + 1024 * i;
    if (c < h) *reinterpret_cast<float4 *>(part + (int64_t)blockIdx.x * h + c) = acc[i];
  }
}

// dg[c] = sum over b < nb of part[b][c]: 64 columns per block, four slices
// of b (b = s, s + 4, ...) summed in order and then added slice by slice.
__global__ __launch_bounds__(256) void rmsnorm_bwd_dg_kernel(const float *__restrict__ part, int32_t nb, int32_t h,
                                                             float *__restrict__ dg) {
  __shared__ float sl[4][64];
  const int col = blockIdx.x * 64 + (threadIdx.x & 63), s = threadIdx.x >> 6;
  float a = 0.f;
  if (col < h)
    for (int b = s; b < nb; b += 4) a += part[(int64_t)b * h + col];
  sl[s][threadIdx.x & 63] = a;
  __syncthreads();
  if (s == 0 && col < h) dg[col] = ((sl[0][threadIdx.x] + sl[1][threadIdx.x]) + sl[2][threadIdx.x]) + sl[3][threadIdx.x];
}

size_t rmsnorm_bwd_part_bytes(int32_t rows, int32_t h) {
  return (size_t)((rows + kNormBwdRows - 1) / kNormBwdRows) * (size_t)h * 4;
}

hipError_t launch_rmsnorm_bwd(const float *x, const void *g, const float *d, const float *res, float *dx, void *lo,
                              bool lo_panel, int32_t rows, int32_t h, float eps, int dtype, float *part, float *dg,
                              hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if ((h & 3) != 0 || h > 4 * 256 * kNormBwdChunks || (h + 63) / 64 > 65535) return hipErrorInvalidValue;
  const int nb = (rows + kNormBwdRows - 1) / kNormBwdRows;
  const int64_t ps = lo_panel ? (int64_t)rows * kPanel : 0;
  if (dtype == TSP_BF16)
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<bf16, bf16>), dim3(nb), dim3(256), 0, s, x, (const bf16 *)g, d, res, dx,
                       (bf16 *)lo, ps, rows, h, eps, part);
  else
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<float, float>), dim3(nb), dim3(256), 0, s, x, (const float *)g, d, res,
                       dx, (float *)lo, (int64_t)0, rows, h, eps, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rmsnorm_bwd_dg_kernel, dim3((h + 63) / 64), dim3(256), 0, s, part, nb, h, dg);
  return hipGetLastError();
}

// ---------------------------------------------------------------- column packing
// out[t][j * (wa + 2 wb) + c] = a[t][j * wa + c] (c < wa), then b[t][j * wb +
// c - wa], then cc[t][j * wb + c - wa - wb], for j < D: fp32 sources
// interleaved by shard into one dtype matrix [n][D (wa + 2 wb)], row-major
// or (bf16) in panel layout. Four consecutive columns never straddle
// sources (wa and wb are multiples of 4). With D = 1 and wb = 0 it is a
// plain conversion of a.
template <typename T>
__global__ __launch_bounds__(256) void pack_cols_kernel(const float *__restrict__ a, const float *__restrict__ b,
                                                        const float *__restrict__ cc, int32_t n, int32_t D,
                                                        int32_t wa, int32_t wb, T *__restrict__ out,
                                                        int64_t out_panel) {
  const int32_t ws = wa + 2 * wb, W = D * ws, W4 = W / 4;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)n * W4) return;
  const int64_t t = e / W4;
  const int32_t col = (int32_t)(e - t * W4) * 4, j = col / ws, c = col - j * ws;
  const float *src;
  if (c < wa)
    src = a + t * ((int64_t)D * wa) + (int64_t)j * wa + c;
  else if (c < wa + wb)
    src = b + t * ((int64_t)D * wb) + (int64_t)j * wb + (c - wa);
  else
    src = cc + t * ((int64_t)D * wb) + (int64_t)j * wb + (c - wa - wb);
  const float4 v = *reinterpret_cast<const float4 *>(src);
  T *o = out + (out_panel ? panel_index(t, col, out_panel) : t * W + col);
  o[0] = (T)v.x;
  o[1] = (T)v.y;
  o[2] = (T)v.z;
  o[3] = (T)v.w;
}

hipError_t launch_pack_cols(int dtype, const float *a, const float *b, const float *c, int32_t n, int32_t D,
                            int32_t wa, int32_t wb, void *out, bool out_panel, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (((wa | wb) & 3) != 0 || (out_panel && dtype != TSP_BF16)) return hipErrorInvalidValue;
  const int64_t total = (int64_t)n * D * (wa + 2 * wb) / 4;
  if ((total + 255) / 256 > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == TSP_BF16)
    hipLaunchKernelGGL(pack_cols_kernel<bf16>, grid, dim3(256), 0, s, a, b, c, n, D, wa, wb, (bf16 *)out,
                       out_panel ? (int64_t)n * kPanel : (int64_t)0);
  else
    hipLaunchKernelGGL(pack_cols_kernel<float>, grid, dim3(256), 0, s, a, b, c, n, D, wa, wb, (float *)out,
                       (int64_t)0);
  return hipGetLastError();
}

// ---------------------------------------------------------------- rotary embedding
// table[t * half + i] = (cos, sin) of pos(t) * base^(-2i/Dh), in fp64 before
// rounding to fp32 (the angle reaches S radians for i = 0).
__global__ __launch_bounds__(256) void rope_table_kernel(ZigzagMap zz, int32_t n, int32_t half, double base,
                                                         float2 *__restrict__ table) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)n * half) return;
  const int t = (int)(e / half), i = (int)(e - (int64_t)t * half);
  const double ang = (double)zz.pos(t) * pow(base, -(double)i / (double)half);
  table[e] = make_float2((float)cos(ang), (float)sin(ang));
}

// In-place rotation of fp32 rows: row t (at x + (scatter ? pos(t) : t) * ld)
// holds H heads of Dh; pair i of a head is features (i, i + Dh/2).
__global__ __launch_bounds__(256) void rope_rows_kernel(float *__restrict__ x, int64_t ld, int32_t n, int32_t H,
                                                        int32_t half, ZigzagMap zz, int32_t scatter,
                                                        const float2 *__restrict__ table) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)n * H * half) return;
  const int t = (int)(e / ((int64_t)H * half));
  const int rem = (int)(e - (int64_t)t * H * half);
  const int hh = rem / half, i = rem - hh * half;
  float *row = x + (int64_t)(scatter ? zz.pos(t) : t) * ld + (int64_t)hh * 2 * half;
  const float2 cs = table[(int64_t)t * half + i];
  const float a = row[i], b = row[i + half];
  row[i] = a * cs.x - b * cs.y;
  row[i + half] = b * cs.x + a * cs.y;
}

hipError_t launch_rope_table(ZigzagMap zz, int32_t n, int32_t Dh, float base, float2 *table, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t total = (int64_t)n * (Dh / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, zz, n, Dh / 2,
                     (double)base, table);
  return hipGetLastError();
}

hipError_t launch_rope_rows(float *x, int64_t ld, int32_t n, int32_t H, int32_t Dh, ZigzagMap zz, bool scatter,
                            const float2 *table, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t total = (int64_t)n * H * (Dh / 2);
  hipLaunchKernelGGL(rope_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, x, ld, n, H, Dh / 2,
                     zz, scatter ? 1 : 0, table);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_f32(const float *x, const void *g, int g_dtype, float *out, int32_t rows, int32_t h,
                              float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (g_dtype == TSP_BF16)
    launch_rmsnorm_rows(x, (const bf16 *)g, out, rows, h, eps, (int64_t)0, s);
  else
    launch_rmsnorm_rows(x, (const float *)g, out, rows, h, eps, (int64_t)0, s);
  return hipGetLastError();
}


// ---------------------------------------------------------------- transpose
// One 256-thread block per 64 x 64 tile of one matrix (blockIdx.z). The tile
// goes through LDS as fp32 (bf16 widens exactly), read along input rows and
// written along output rows, so both sides are contiguous runs of 64
// elements (a panel layout keeps 64 aligned columns contiguous too). The
// padded LDS row keeps the column reads conflict-free.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(PtrList in, int64_t in_ld, int64_t in_panel, int32_t R,
                                                        int32_t C, T *__restrict__ out, int64_t out_ld,
                                                        int64_t out_panel, int64_t out_zoff) {
  __shared__ float tile[64][65];
  const T *src = reinterpret_cast<const T *>(in.p[blockIdx.z]);
  T *dst = out + (int64_t)blockIdx.z * out_zoff;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + ty + 4 * i, c = c0 + tx;
    float v = 0.f;
    if (r < R && c < C) v = (float)src[in_panel ? panel_index(r, c, in_panel) : (int64_t)r * in_ld + c];
    tile[ty + 4 * i][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = c0 + ty + 4 * i, r = r0 + tx;  // output row c, column r
    if (r < R && c < C) dst[out_panel ? panel_index(c, r, out_panel) : (int64_t)c * out_ld + r] = (T)tile[tx][ty + 4 * i];
  }
}

// bf16 with R and C multiples of 8: each thread moves 16-byte runs (8
// elements) both ways, through a 64 x 64 tile with rows padded by 16 bytes.
__global__ __launch_bounds__(256) void transpose_bf16x8_kernel(PtrList in, int64_t in_ld, int64_t in_panel, int32_t R,
                                                               int32_t C, bf16 *__restrict__ out, int64_t out_ld,
                                                               int64_t out_panel, int64_t out_zoff) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][72];
  const bf16 *src = reinterpret_cast<const bf16 *>(in.p[blockIdx.z]);
  bf16 *dst = out + (int64_t)blockIdx.z * out_zoff;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int chunk = threadIdx.x + 256 * i, row = chunk >> 3, cc = (chunk & 7) * 8;
    const int r = r0 + row, c = c0 + cc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4 *>(src + (in_panel ? panel_index(r, c, in_panel) : (int64_t)r * in_ld + c));
    *reinterpret_cast<u32x4 *>(&tile[row][cc]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int chunk = threadIdx.x + 256 * i, orow = chunk >> 3, oc = (chunk & 7) * 8;  // output row c0 + orow
    const int c = c0 + orow, r = r0 + oc;
    if (c < C && r < R) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[oc + e][orow];
      *reinterpret_cast<bf16x8 *>(dst + (out_panel ? panel_index(c, r, out_panel) : (int64_t)c * out_ld + r)) = v;
    }
  }
}

// Z [R = n][C = F] to Z^T (panels of [F][n]) and GELU(Z)^T ([F][n] row-major),
// 16-byte runs through a padded 64 x 64 tile as in transpose_bf16x8_kernel.
__global__ __launch_bounds__(256) void transpose_gelu_kernel(const bf16 *__restrict__ z, int32_t R, int32_t C,
                                                             bf16 *__restrict__ zt, bf16 *__restrict__ ht) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][72];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int64_t zt_panel = (int64_t)C * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int chunk = threadIdx.x + 256 * i, row = chunk >> 3, cc = (chunk & 7) * 8;
    const int r = r0 + row, c = c0 + cc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4 *>(z + (int64_t)r * C + c);
    *reinterpret_cast<u32x4 *>(&tile[row][cc]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int chunk = threadIdx.x + 256 * i, orow = chunk >> 3, oc = (chunk & 7) * 8;
    const int c = c0 + orow, r = r0 + oc;
    if (c < C && r < R) {
      bf16x8 v, gv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = tile[oc + e][orow];
        gv[e] = (bf16)gelu_erf((float)v[e]);
      }
      *reinterpret_cast<bf16x8 *>(zt + panel_index(c, r, zt_panel)) = v;
      *reinterpret_cast<bf16x8 *>(ht + (int64_t)c * R + r) = gv;
    }
  }
}

hipError_t launch_transpose_gelu(const void *z, int32_t n, int32_t F, void *zt_panel, void *ht, hipStream_t s) {
  if (n <= 0 || F <= 0) return hipSuccess;
  if (((n | F) & 7) != 0 || (n + 63) / 64 > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_gelu_kernel, dim3((F + 63) / 64, (n + 63) / 64), dim3(256), 0, s,
                     reinterpret_cast<const bf16 *>(z), n, F, reinterpret_cast<bf16 *>(zt_panel),
                     reinterpret_cast<bf16 *>(ht));
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, const PtrList &in, int32_t nz, int64_t in_ld, int64_t in_panel, int32_t R,
                            int32_t C, void *out, int64_t out_ld, int64_t out_panel, int64_t out_zoff, hipStream_t s) {
  if (R <= 0 || C <= 0 || nz <= 0) return hipSuccess;
  if ((in_panel || out_panel) && dtype != TSP_BF16) return hipErrorInvalidValue;
  if (nz > TSP_MAX_D || (R + 63) / 64 > 65535) return hipErrorInvalidValue;
  const dim3 grid((C + 63) / 64, (R + 63) / 64, nz);
  // 16-byte runs need 8-element alignment of both extents, pitches and offsets
  const bool x8 = ((R | C) & 7) == 0 && (in_ld & 7) == 0 && (out_ld & 7) == 0 && (out_zoff & 7) == 0;
  if (dtype == TSP_BF16 && x8)
    hipLaunchKernelGGL(transpose_bf16x8_kernel, grid, dim3(256), 0, s, in, in_ld, in_panel, R, C,
                       reinterpret_cast<bf16 *>(out), out_ld, out_panel, out_zoff);
  else if (dtype == TSP_BF16)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, s, in, in_ld, in_panel, R, C,
                       reinterpret_cast<bf16 *>(out), out_ld, out_panel, out_zoff);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, in, in_ld, in_panel, R, C,
                       reinterpret_cast<float *>(out), out_ld, out_panel, out_zoff);
  return hipGetLastError();
}

}  // namespace tsp
