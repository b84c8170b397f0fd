// Shard-wise GEMMs of the layer: C = A B^T with A [M][K] and B [N][K], both
// contiguous along K, fp32 accumulation, and a fused epilogue per use:
//   QKV      : scatter Q to the local Q buffer and K/V to their global rows
//   out-proj : reduction walks the D W_O shards in broadcast order, + residual
//   MLP up   : exact GELU, stored in the operand dtype
//   MLP down : fp32 store / accumulate into the residual stream
//
// bf16 operands run on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16):
// a 256x256 block tile, 8 waves as 2 (M) x 4 (N), each wave owning 128x64 of
// the output as 4x2 MFMA accumulators of 32x32. K advances 64 at a time
// through two LDS stages; the next stage's global loads are issued before the
// current stage's MFMAs so their latency is covered, and one barrier per step
// separates the stages. LDS rows are 128 bytes (64 bf16) with the 16-byte
// chunk index XOR-swizzled by (row/2)%8, so the 16 lanes that share a bank
// window read 16 different bank groups.
// fp32 operands use a plain LDS-tiled FMA kernel (64x64 tiles, 4x4 per thread).
#include "device_common.h"
#include "tsp_internal.h"

namespace tsp {

struct GemmArgs {
  const void *A;  // [M][K_total] (lda elements per row)
  int64_t lda;
  PtrList B;      // B segments: segment s holds columns [s*kseg, (s+1)*kseg) of B
  int64_t ldb;    // row pitch of every B segment
  int32_t kseg;   // reduction length covered by one B pointer
  int32_t M, N, K;
  int32_t nz;     // independent problems; problem z uses B.p[z] and K == kseg
};

// ---------------------------------------------------------------- epilogues
template <typename T>
struct EpiGelu {
  T *out;
  int64_t ld;
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const {
    out[(int64_t)r * ld + c] = (T)gelu_erf(v);
  }
};

struct EpiStoreF32 {
  float *out;
  int64_t ld;
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const { out[(int64_t)r * ld + c] = v; }
};

// out = res + v; res may alias out (each element is read then written by the
// same lane).
struct EpiAddF32 {
  const float *res;
  float *out;
  int64_t ld;
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const {
    const int64_t i = (int64_t)r * ld + c;
    out[i] = res[i] + v;
  }
};

// Shard z of the QKV projection: output column c of the shard falls in part
// c / hd (0 = Q, 1 = K, 2 = V), head-group feature c % hd, i.e. global feature
// z*hd + c % hd. Q stays in local row order; K and V go to the global row of
// the token.
template <typename T>
struct EpiQKV {
  T *q, *k, *v;
  int64_t h;
  int32_t hd;
  ZigzagMap zz;
  __device__ __forceinline__ void operator()(int z, int r, int c, float val) const {
    const int part = c / hd;
    const int64_t col = (int64_t)z * hd + (c - part * hd);
    if (part == 0) {
      q[(int64_t)r * h + col] = (T)val;
    } else {
      T *dst = part == 1 ? k : v;
      dst[(int64_t)zz.pos(r) * h + col] = (T)val;
    }
  }
};

// ---------------------------------------------------------------- tile order
// Logical tile L -> (z, tm, tn): problems outermost, then groups of GM tile
// rows walked column-major, so the blocks that run together on one XCD share
// A row panels and B column panels in its L2.
struct TileCoord {
  int z, tm, tn;
};
__device__ __forceinline__ TileCoord tile_of(int L, int tiles_m, int tiles_n) {
  constexpr int GM = 8;
  const int per_z = tiles_m * tiles_n;
  TileCoord t;
  t.z = L / per_z;
  const int rem = L - t.z * per_z;
  const int group = rem / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = rem - group * GM * tiles_n;
  t.tm = first_m + in_group % gsize;
  t.tn = in_group / gsize;
  return t;
}

// ---------------------------------------------------------------- bf16 MFMA
constexpr int kBM = 256, kBN = 256, kBK = 64, kGemmThreads = 512;
constexpr int kStageElems = (kBM + kBN) * kBK;  // bf16 elements per LDS stage
constexpr size_t kGemmLds = 2 * kStageElems * sizeof(bf16);

__device__ __forceinline__ int swz_off(int row, int chunk) {  // element offset in a 64-wide row
  return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

template <class Epi>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(GemmArgs a, Epi epi) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16 *smem = reinterpret_cast<bf16 *>(smem_raw);

  const int tiles_m = (a.M + kBM - 1) / kBM, tiles_n = (a.N + kBN - 1) / kBN;
  const TileCoord tc = tile_of(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n);
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN, z = tc.z;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;

  const bf16 *A = reinterpret_cast<const bf16 *>(a.A);
  const int ld_row = tid >> 3, ld_ch = tid & 7;  // loader: rows ld_row + 64*i, chunk ld_ch

  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * kBK;
    int seg, koff;
    if (a.nz > 1) {
      seg = z;
      koff = k0;
    } else {
      seg = k0 / a.kseg;
      koff = k0 - seg * a.kseg;
    }
    const bf16 *B = reinterpret_cast<const bf16 *>(a.B.p[seg]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = ld_row + 64 * i;
      const int gm = m0 + row, gn = n0 + row;
      u32x4 zero = {0u, 0u, 0u, 0u};
      ra[i] = gm < a.M ? *reinterpret_cast<const u32x4 *>(A + (int64_t)gm * a.lda + k0 + ld_ch * 8) : zero;
      rb[i] = gn < a.N ? *reinterpret_cast<const u32x4 *>(B + (int64_t)gn * a.ldb + koff + ld_ch * 8) : zero;
    }
  };
  auto sstore = [&](int buf) {
    bf16 *As = smem + buf * kStageElems;
    bf16 *Bs = As + kBM * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = ld_row + 64 * i;
      *reinterpret_cast<u32x4 *>(As + swz_off(row, ld_ch)) = ra[i];
      *reinterpret_cast<u32x4 *>(Bs + swz_off(row, ld_ch)) = rb[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = a.K / kBK;
  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const bf16 *As = smem + cur * kStageElems;
    const bf16 *Bs = As + kBM * kBK;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8 *>(As + swz_off(row, ch));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8 *>(Bs + swz_off(row, ch));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // accumulator layout of a 32x32 MFMA: lane holds column lane%32 and rows
  // 8*(v/4) + 4*(lane/32) + v%4 for v = 0..15
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= a.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (row < a.M) epi(z, row, col, acc[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------- fp32 FMA
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a, Epi epi) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const TileCoord tc = tile_of(blockIdx.x, tiles_m, tiles_n);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN, z = tc.z;
  const float *A = reinterpret_cast<const float *>(a.A);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += BK) {
    int seg, koff;
    if (a.nz > 1) {
      seg = z;
      koff = k0;
    } else {
      seg = k0 / a.kseg;
      koff = k0 - seg * a.kseg;
    }
    const float *B = reinterpret_cast<const float *>(a.B.p[seg]);
    float4 av = make_float4(0.f, 0.f, 0.f, 0.f), bv = av;
    if (m0 + lrow < a.M) av = *reinterpret_cast<const float4 *>(A + (int64_t)(m0 + lrow) * a.lda + k0 + lk);
    if (n0 + lrow < a.N) bv = *reinterpret_cast<const float4 *>(B + (int64_t)(n0 + lrow) * a.ldb + koff + lk);
    As[lk + 0][lrow] = av.x;
    As[lk + 1][lrow] = av.y;
    As[lk + 2][lrow] = av.z;
    As[lk + 3][lrow] = av.w;
    Bs[lk + 0][lrow] = bv.x;
    Bs[lk + 1][lrow] = bv.y;
    Bs[lk + 2][lrow] = bv.z;
    Bs[lk + 3][lrow] = bv.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float ar[4], br[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ar[i] = As[k][ty * 4 + i];
        br[i] = Bs[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = m0 + ty * 4 + i, c = n0 + tx * 4 + j;
      if (r < a.M && c < a.N) epi(z, r, c, acc[i][j]);
    }
}

// ---------------------------------------------------------------- launchers
template <class Epi>
static hipError_t run_gemm(int dtype, const GemmArgs &a, const Epi &epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (dtype == TSP_BF16) {
    static bool attr_set = false;  // benign race: every caller sets the same value
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_bf16_kernel<Epi>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    const int tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN) * a.nz;
    hipLaunchKernelGGL((gemm_bf16_kernel<Epi>), dim3(tiles), dim3(kGemmThreads), kGemmLds, s, a, epi);
  } else {
    const int tiles = ((a.M + 63) / 64) * ((a.N + 63) / 64) * a.nz;
    hipLaunchKernelGGL((gemm_f32_kernel<Epi>), dim3(tiles), dim3(256), 0, s, a, epi);
  }
  return hipGetLastError();
}

static GemmArgs make_args(const void *A, int64_t lda, int32_t M, int32_t N, int32_t K) {
  GemmArgs a{};
  a.A = A;
  a.lda = lda;
  a.M = M;
  a.N = N;
  a.K = K;
  a.kseg = K;
  a.nz = 1;
  return a;
}

hipError_t launch_qkv(int dtype, const void *xn, int32_t n, int32_t h, const PtrList &w, int32_t D,
                      int32_t hd, void *q, void *kf, void *vf, ZigzagMap zz, hipStream_t s) {
  GemmArgs a = make_args(xn, h, n, 3 * hd, h);
  a.B = w;
  a.ldb = h;
  a.nz = D;
  if (dtype == TSP_BF16) {
    EpiQKV<bf16> e{(bf16 *)q, (bf16 *)kf, (bf16 *)vf, h, hd, zz};
    return run_gemm(dtype, a, e, s);
  }
  EpiQKV<float> e{(float *)q, (float *)kf, (float *)vf, h, hd, zz};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_outproj(int dtype, const void *o, int32_t n, int32_t h, const PtrList &wo, int32_t D,
                          int32_t hd, const float *x, float *y, hipStream_t s) {
  GemmArgs a = make_args(o, h, n, h, D * hd);
  a.B = wo;
  a.ldb = hd;
  a.kseg = hd;
  EpiAddF32 e{x, y, h};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_mlp_up(int dtype, const void *x, int32_t n, int32_t h, const void *w1j, int32_t fd,
                         void *hid, hipStream_t s) {
  GemmArgs a = make_args(x, h, n, fd, h);
  a.B.p[0] = w1j;
  a.ldb = h;
  if (dtype == TSP_BF16) {
    EpiGelu<bf16> e{(bf16 *)hid, fd};
    return run_gemm(dtype, a, e, s);
  }
  EpiGelu<float> e{(float *)hid, fd};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_mlp_down(int dtype, const void *hid, int32_t n, int32_t fd, const void *w2j, int32_t h,
                           const float *res, float *y, hipStream_t s) {
  GemmArgs a = make_args(hid, fd, n, h, fd);
  a.B.p[0] = w2j;
  a.ldb = fd;
  if (res) {
    EpiAddF32 e{res, y, h};
    return run_gemm(dtype, a, e, s);
  }
  EpiStoreF32 e{y, h};
  return run_gemm(dtype, a, e, s);
}

}  // namespace tsp
