// Shard-wise GEMMs of the layer: C = A B^T with A [M][K] and B [N][K], both
// contiguous along K, fp32 accumulation, and a fused epilogue per use:
//   QKV      : all D attention shards in one launch (shard = grid problem);
//              Q to the local Q buffer, K/V to their global rows
//   out-proj : the reduction walks the D W_O shards in broadcast order, + x
//   MLP up   : all D ring shards in one launch, exact GELU, stored in the
//              operand dtype at the shard's ring-step columns of H
//   MLP down : the reduction walks H and the D W2 shards in ring order, + h1
//
// bf16 operands run on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
// Block tile 256 (M) x 256 (N), 8 waves as 4 (M) x 2 (N), each wave owning
// 64 x 128 of the output as 2 x 4 MFMA accumulators of 32 x 32. The MFMAs
// produce C^T blocks (B rows are the first operand), so a lane holds 4
// consecutive output columns of one row and every epilogue access is a 16-
// (fp32) or 8-byte (bf16) vector.
// K advances 32 at a time through a ring of 4 LDS stages (A and B tiles of
// 256 x 32, 32 KB per stage, 128 KB): tiles go from HBM straight into LDS
// (buffer_load ... lds, 16 bytes per lane) three steps ahead of their use,
// one block barrier per step. LDS rows are 64 bytes; the 16-byte chunk index
// is XOR-swizzled by (row/4)%4 (the copying lane picks its source chunk), so
// the 16 lanes that read one chunk of 16 rows hit 16 distinct bank groups.
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
// Each epilogue takes one output element (fp32 kernel) or four consecutive
// columns of one row (bf16 kernel) of problem z.
template <typename T>
__device__ __forceinline__ void store4(T *p, float4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4 *>(p) = v;
  } else {
    const bf16x2 lo = {(bf16)v.x, (bf16)v.y}, hi = {(bf16)v.z, (bf16)v.w};
    u32x2 u = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    *reinterpret_cast<u32x2 *>(p) = u;
  }
}

// H[:, z*cols + c] = GELU(acc): problem z is ring step z's shard.
template <typename T>
struct EpiGelu {
  T *out;
  int64_t ld;    // row pitch of H
  int32_t cols;  // columns per shard
  __device__ __forceinline__ void operator()(int z, int r, int c, float v) const {
    out[(int64_t)r * ld + (int64_t)z * cols + c] = (T)gelu_erf(v);
  }
  __device__ __forceinline__ void operator()(int z, int r, int c, float4 v) const {
    store4(out + (int64_t)r * ld + (int64_t)z * cols + c,
           make_float4(gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w)));
  }
};

struct EpiStoreF32 {
  float *out;
  int64_t ld;
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const { out[(int64_t)r * ld + c] = v; }
  __device__ __forceinline__ void operator()(int, int r, int c, float4 v) const {
    *reinterpret_cast<float4 *>(out + (int64_t)r * ld + c) = v;
  }
};

// out = res + acc; res may alias out (each element is read then written by
// the same lane).
struct EpiAddF32 {
  const float *res;
  float *out;
  int64_t ld;
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const {
    const int64_t i = (int64_t)r * ld + c;
    out[i] = res[i] + v;
  }
  __device__ __forceinline__ void operator()(int, int r, int c, float4 v) const {
    const int64_t i = (int64_t)r * ld + c;
    const float4 x = *reinterpret_cast<const float4 *>(res + i);
    *reinterpret_cast<float4 *>(out + i) = make_float4(x.x + v.x, x.y + v.y, x.z + v.z, x.w + v.w);
  }
};

// Shard z of the QKV projection: output column c of the shard falls in part
// c / hd (0 = Q, 1 = K, 2 = V), head-group feature c % hd, i.e. global feature
// z*hd + c % hd. Q stays in local row order; K and V go to the global row of
// the token. (Four consecutive columns never straddle parts: hd % 4 == 0.)
template <typename T>
struct EpiQKV {
  T *q, *k, *v;
  int64_t h;
  int32_t hd;
  ZigzagMap zz;
  __device__ __forceinline__ T *dst(int z, int r, int c) const {
    const int part = c / hd;
    const int64_t col = (int64_t)z * hd + (c - part * hd);
    if (part == 0) return q + (int64_t)r * h + col;
    return (part == 1 ? k : v) + (int64_t)zz.pos(r) * h + col;
  }
  __device__ __forceinline__ void operator()(int z, int r, int c, float val) const { *dst(z, r, c) = (T)val; }
  __device__ __forceinline__ void operator()(int z, int r, int c, float4 val) const { store4(dst(z, r, c), val); }
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
constexpr int kBM = 256, kBN = 256, kBK = 32, kGemmThreads = 512, kGemmStages = 4;
constexpr int kTileBytes = kBM * kBK * 2;                       // one 256 x 32 bf16 tile: 16 KB
constexpr int kGemmStageBytes = 2 * kTileBytes;                 // A tile + B tile
constexpr size_t kGemmLds = (size_t)kGemmStages * kGemmStageBytes;  // 128 KB
constexpr int kGemmLoads = 4;  // copy instructions per wave per K step

// Byte offset of logical 16-byte chunk ch (0..3) of row r in a 64-byte-row tile.
__device__ __forceinline__ int gswz(int r, int ch) { return r * 64 + ((ch ^ ((r >> 2) & 3)) << 4); }

template <class Epi>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(GemmArgs a, Epi epi) {
#if defined(__HIP_DEVICE_COMPILE__)
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tiles_m = (a.M + kBM - 1) / kBM, tiles_n = (a.N + kBN - 1) / kBN;
  const TileCoord tc = tile_of(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n);
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN, z = tc.z;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // wave tile: rows wm*64.., columns wn*128..
  const int g = lane >> 5, l32 = lane & 31;

  // ---- copy plan: each wave copies A windows 2*wave, 2*wave+1 and the same B
  // windows of every stage; window w = tile rows 16w..16w+15 (1 KB). Lane ->
  // (row, chunk position); it loads the logical chunk that belongs there.
  const uint32_t lds0 = lds_addr(smem);
  int a_off[2], b_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int win = 2 * wave + i, row = win * 16 + lane / 4, pos = lane & 3;
    const int ch = pos ^ ((row >> 2) & 3);
    a_off[i] = (int)(row * a.lda * 2) + ch * 16;
    b_off[i] = (int)(row * a.ldb * 2) + ch * 16;
  }
  const int a_rows = min(kBM, a.M - m0), b_rows = min(kBN, a.N - n0);
  const bf16 *Ab = reinterpret_cast<const bf16 *>(a.A) + (int64_t)m0 * a.lda;
  const u32x4 ar = buffer_rsrc(Ab, (uint32_t)(a_rows * a.lda * 2));
  auto copy_step = [&](int kt, int st) {
    const int k0 = kt * kBK;
    int seg, koff;
    if (a.nz > 1) {
      seg = z;
      koff = k0;
    } else {
      seg = k0 / a.kseg;
      koff = k0 - seg * a.kseg;
    }
    const bf16 *Bb = reinterpret_cast<const bf16 *>(a.B.p[seg]) + (int64_t)n0 * a.ldb;
    const u32x4 br = buffer_rsrc(Bb, (uint32_t)(b_rows * a.ldb * 2));
    const uint32_t base = lds0 + st * kGemmStageBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t win = 2 * wave + i;
      lds_copy16(ar, a_off[i], k0 * 2, base + win * 1024);
      lds_copy16(br, b_off[i], koff * 2, base + kTileBytes + win * 1024);
    }
  };

  // fragment read offsets inside a stage: A rows wm*64 + j*32 + l32, B rows
  // wn*128 + i*32 + l32; chunk 2*kk + g of the 32-wide K step
  int fa_a[2][2], fa_b[4][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int j = 0; j < 2; ++j) fa_a[j][kk] = gswz(wm * 64 + j * 32 + l32, 2 * kk + g);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa_b[i][kk] = kTileBytes + gswz(wn * 128 + i * 32 + l32, 2 * kk + g);
  }

  f32x16 acc[4][2];  // acc[i][j]: C^T block (N block i, M block j)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = a.K / kBK;
  // prologue: steps 0..2 in flight; step 0 landed before the first barrier
  for (int p = 0; p < kGemmStages - 1 && p < KT; ++p) copy_step(p, p);
  if (KT >= 3)
    wait_vmcnt<2 * kGemmLoads>();
  else if (KT == 2)
    wait_vmcnt<kGemmLoads>();
  else
    wait_vmcnt<0>();
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    // stage (kt+3)%4 last held step kt-1, which every wave finished before the
    // barrier that ended it
    if (kt + 3 < KT) copy_step(kt + 3, (kt + 3) % kGemmStages);
    const unsigned char *st = smem + (kt % kGemmStages) * kGemmStageBytes;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 af[2], bfr[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) af[j] = *reinterpret_cast<const bf16x8 *>(st + fa_a[j][kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i) bfr[i] = *reinterpret_cast<const bf16x8 *>(st + fa_b[i][kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[i], af[j], acc[i][j], 0, 0, 0);
    }
    // step kt+1 must have landed (this wave's copies) before the barrier;
    // the copies of steps kt+2 and kt+3 may stay in flight
    if (kt + 3 < KT)
      wait_vmcnt<2 * kGemmLoads>();
    else if (kt + 2 < KT)
      wait_vmcnt<kGemmLoads>();
    else
      wait_vmcnt<0>();
    __syncthreads();
  }

  // accumulator layout (C^T block): lane holds output row (M) l32 of the
  // block and columns (N) 8*(v/4) + 4*g + v%4
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = m0 + wm * 64 + j * 32 + l32;
    if (row >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int col = n0 + wn * 128 + i * 32 + vq * 8 + g * 4;
        if (col < a.N)
          epi(z, row, col,
              make_float4(acc[i][j][vq * 4 + 0], acc[i][j][vq * 4 + 1], acc[i][j][vq * 4 + 2], acc[i][j][vq * 4 + 3]));
      }
  }
#endif  // __HIP_DEVICE_COMPILE__
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

hipError_t launch_mlp_up(int dtype, const void *x, int32_t n, int32_t h, const PtrList &w1, int32_t D, int32_t fd,
                         void *hid, hipStream_t s) {
  GemmArgs a = make_args(x, h, n, fd, h);
  a.B = w1;
  a.ldb = h;
  a.nz = D;
  if (dtype == TSP_BF16) {
    EpiGelu<bf16> e{(bf16 *)hid, (int64_t)D * fd, fd};
    return run_gemm(dtype, a, e, s);
  }
  EpiGelu<float> e{(float *)hid, (int64_t)D * fd, fd};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_mlp_down(int dtype, const void *hid, int32_t n, const PtrList &w2, int32_t D, int32_t fd,
                           int32_t h, const float *res, float *y, hipStream_t s) {
  GemmArgs a = make_args(hid, (int64_t)D * fd, n, h, D * fd);
  a.B = w2;
  a.ldb = fd;
  a.kseg = fd;
  if (res) {
    EpiAddF32 e{res, y, h};
    return run_gemm(dtype, a, e, s);
  }
  EpiStoreF32 e{y, h};
  return run_gemm(dtype, a, e, s);
}

}  // namespace tsp
