// Backward of the zigzag causal attention on one rank: the gradients of the
// rank's queries (dQ) and the rank's contribution to the gradients of every
// key and value row of the gathered sequence (dK, dV), from the output
// gradient dO. With P = softmax(scale * Q K^T) over the visible keys and
// dP = dO V^T, the softmax Jacobian gives dS = P * (dP - Delta), Delta the row
// sum of dO * O; then dQ = scale * dS K, dK = scale * dS^T Q, dV = P^T dO.
//
// Two launches:
//  1. dQ, query-major (like the forward): block = 4 waves x 32 queries of one
//     head. A first walk over the key tiles takes each row's log-sum-exp and
//     Delta = sum_u P_u dP_u (S^T = K Q^T and dP^T = V dO^T, a lane owning one
//     query and 32 of a tile's keys; both kept for launch 2). Delta is formed
//     from the fp32 probabilities rather than from a stored bf16 O, whose
//     rounding would pass into every dS of rows that see few keys. A second
//     walk recomputes S^T and dP^T, forms dS^T and accumulates dQ^T += K^T
//     dS^T. The K^T operand comes from transpose reads of a second copy of the
//     K tile, laid out for them.
//  2. dK and dV, key-major: block = 4 waves x 32 keys of one K/V head. It walks
//     the rank's query rows that can see its keys, 32 at a time (staged into
//     LDS 64 at a time), over every query head that reads the K/V head:
//     S = Q K^T and dP = dO V^T with the keys on the lanes, P and dS from
//     the row statistics of launch 1, then
//     dV^T += dO^T P and dK^T += Q^T dS, whose dO^T and Q^T operands are
//     transpose reads of the query tiles.
// When the forward's fp32 O and log-sum-exp are given, a small kernel forms
// Delta = rowsum(dO * O) and the log2-domain statistics instead, and a dQ
// kernel without the first walk (attn_bwd_dq_lds_kernel) stages its K/V tiles
// the way the forward does: straight into LDS, double-buffered.
// The operands of the second products are the score registers themselves,
// rounded to bf16, in the order the MFMA takes them; the transpose reads hand
// each lane 4 consecutive rows of one feature in that order. Every product
// runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation. SPLIT: P and dS
// enter their products as a bf16 pair hi + lo (two MFMAs each), exact to
// about 2^-16 of their size: a plain bf16 rounding (2^-9) of them leaves
// elements off by 2-4% of the tensor's rms gradient on ranks whose rows see
// thousands of keys (the largest gradient rows carry the error), not only
// on the first rows of the sequence as in the forward. Without SPLIT they
// enter rounded once to bf16, one MFMA each, as in common flash-attention
// backward kernels; norm-wise the error stays near the bf16 rounding unit.
//
// fp32 inputs run plain per-row kernels with exact expf.
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "tsp_internal.h"

namespace tsp {

struct BwdArgs {
  const void *q, *k, *v, *dout;
  const float *o_f32, *lse_in;  // the forward's fp32 O and natural log-sum-exp, or null
  float *dq, *dk, *dv;
  float *lse;    // [H][n]: log2 of each row's softmax denominator (scores in the log2 domain)
  float *delta;  // [H][n]: sum over the row's keys of P dP
  int64_t S;
  int32_t n, H, Hkv, grp;
  float scale, c;  // c = scale * log2(e) (at least the smallest normal float); 1 with pre-scaled q
  float dk_scale;  // multiplier of dK: scale, or ln 2 with pre-scaled q (dK = ln 2 * dS^T q')
  ZigzagMap zz;
  int32_t Tq;  // 128-row query tiles per chunk (dQ kernel)
  int32_t Tk;  // 128-key tiles over the sequence (dK/dV kernel)
};

typedef short s16x4_b __attribute__((ext_vector_type(4)));

// Geometry of an R x DH bf16 tile in LDS: row-major, 16-byte chunks XOR-
// swizzled by row, for ds_read_b128 row fragments and, read transposed, for
// the 4 x 4 transpose reads; both free of bank conflicts: the 16 rows of a
// row read get 16 (DH 128) or 8 pairs of (DH 64) distinct chunk positions,
// and the four rows 4k..4k+3 of a transpose read, which take 2 or 4
// neighbouring chunks each, get disjoint ones. The swizzle depends on the
// row modulo 16 only.
template <int DH>
struct BTile {
  static constexpr int ROWB = DH * 2;
  static constexpr int CPR = DH / 8;
  static __device__ __forceinline__ int row_swz(int row, int ch) {
    return ch ^ (CPR == 16 ? (((row & 3) << 2) | ((row >> 2) & 3))
                           : (((row >> 1) & 3) | ((((row >> 1) ^ (row >> 3)) & 1) << 2)));
  }
};

// R rows of a bf16 [*][pitch] tensor (DH columns) go to LDS in ROW or TR
// layout in two halves, so that the global loads of the next tile can be
// issued before the current tile's math and land in registers meanwhile:
// load_tile_buf fills this thread's chunks, store_tile writes them to LDS.
template <int DH, int R>
struct TileRegs {
  static constexpr int N = R * BTile<DH>::CPR / 256;  // 16-byte chunks per thread
  u32x4 v[N];
};
// Rows [0, nvalid) are read from src (its first row); the rest come back as
// zeros from the buffer descriptor's range, so the loads need no per-lane
// branch and no 64-bit address arithmetic.
template <int DH, int R>
__device__ __forceinline__ void load_tile_buf(TileRegs<DH, R> &t, const bf16 *src, int pitch, int nvalid) {
  using G = BTile<DH>;
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, nvalid * pitch * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < TileRegs<DH, R>::N; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / G::CPR, ch = c % G::CPR;
    t.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, row * pitch * 2 + ch * 16, 0, 0));
  }
}
template <int DH, int R>
__device__ __forceinline__ void store_tile(unsigned char *dst, const TileRegs<DH, R> &t) {
  using G = BTile<DH>;
#pragma unroll
  for (int i = 0; i < TileRegs<DH, R>::N; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / G::CPR, ch = c % G::CPR;
    *reinterpret_cast<u32x4 *>(dst + row * G::ROWB + G::row_swz(row, ch) * 16) = t.v[i];
  }
}

// Lane-constant LDS byte offsets of the fragment reads of a tile, computed
// once per kernel. row[kk]: the chunk of row lane%32, logical chunk 2*kk +
// lane/32; rows 32.. are 32*ROWB further (same swizzle, which depends on the
// row modulo 16). tr[db][hv]: the transpose read that gives lane l feature
// 32*db + l%32's rows 8*hv + 4*(l/32) + {0..3}; rows 16*s.. of a step s of 16
// rows are 16*s*ROWB further (the swizzle again repeats every 16 rows).
template <int DH>
struct FragOff {
  int row[DH / 16];
  int tr[DH / 32][2];
};
template <int DH>
__device__ __forceinline__ FragOff<DH> frag_off(int lane) {
  using G = BTile<DH>;
  FragOff<DH> f;
  const int g = lane >> 5, l32 = lane & 31, r16 = lane & 15, dsub = (lane >> 4) & 1;
#pragma unroll
  for (int kk = 0; kk < DH / 16; ++kk) f.row[kk] = l32 * G::ROWB + G::row_swz(l32, 2 * kk + g) * 16;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      const int row = 8 * hv + g * 4 + (r16 >> 2);
      const int dstart = db * 32 + dsub * 16 + 4 * (r16 & 3);
      f.tr[db][hv] = row * G::ROWB + G::row_swz(row, dstart >> 3) * 16 + (dstart & 7) * 2;
    }
  return f;
}

// Row fragment (ROW layout) at a precomputed offset.
__device__ __forceinline__ bf16x8 row_frag(const unsigned char *t, int off) {
  return *reinterpret_cast<const bf16x8 *>(t + off);
}

// Transpose fragment of a row-layout tile: lane l receives, for feature
// 32*db + l%32, rows 16*st + 4*(l/32) + {0..3} and 16*st + 8 + 4*(l/32) +
// {0..3}: the A operand whose k index runs over those rows in the order of
// the score registers.
template <int DH>
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char *t, const FragOff<DH> &fo, int db, int st) {
  s16x4_b part[2];
#pragma unroll
  for (int hv = 0; hv < 2; ++hv)
    part[hv] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_b *)(t + fo.tr[db][hv] + st * 16 * BTile<DH>::ROWB));
  const s16x8_t both = {part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
  return __builtin_bit_cast(bf16x8, both);
}

// ---------------------------------------------------------------- dQ (bf16)
constexpr int kBwdKey = 64;  // keys per tile of the dQ walk

// v0, v1 as bf16 at elements e, e + 1 of hi (one packed conversion), and
// the remainders v - hi (exact in fp32) as bf16 at the same elements of lo.
// Without SPLIT only hi is written.
template <bool SPLIT>
__device__ __forceinline__ void put_split2(bf16x8 &hi, bf16x8 &lo, int e, float v0, float v1) {
  const bf16x2 h = {(bf16)v0, (bf16)v1};
  hi[e] = h[0];
  hi[e + 1] = h[1];
  if constexpr (SPLIT) {
    const bf16x2 l = {(bf16)(v0 - (float)h[0]), (bf16)(v1 - (float)h[1])};
    lo[e] = l[0];
    lo[e + 1] = l[1];
  }
}

// Row statistics from the forward: Delta = sum over features of dO * O
// (fp32 O) and the log-sum-exp in the log2 domain, one thread per (row,
// head), head fastest.
__global__ __launch_bounds__(256) void attn_bwd_stats_kernel(BwdArgs a, int DH) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.n * a.H) return;
  const int64_t row = i / a.H;
  const int head = (int)(i - row * a.H);
  const float4 *o = reinterpret_cast<const float4 *>(a.o_f32 + i * DH);
  const bf16 *d = reinterpret_cast<const bf16 *>(a.dout) + i * DH;
  float acc = 0.f;
  for (int e = 0; e < DH / 4; ++e) {
    const float4 ov = o[e];
    acc = fmaf(ov.x, (float)d[4 * e], acc);
    acc = fmaf(ov.y, (float)d[4 * e + 1], acc);
    acc = fmaf(ov.z, (float)d[4 * e + 2], acc);
    acc = fmaf(ov.w, (float)d[4 * e + 3], acc);
  }
  const int64_t at = (int64_t)head * a.n + row;
  a.delta[at] = acc;
  a.lse[at] = a.lse_in[at] * 1.4426950408889634f;
}

// Two waves per SIMD (two blocks per CU): the register budget of 256 costs a
// few spilled registers at Dh = 128, which the second wave more than repays.
template <int DH, bool SPLIT>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using G = BTile<DH>;
  constexpr int ND = DH / 32, NK = DH / 16;
  constexpr int TB = kBwdKey * G::ROWB;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][TB];  // K, V (row layout)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const FragOff<DH> fo = frag_off<DH>(lane);
  const int head = blockIdx.x / (2 * a.Tq), tile = blockIdx.x % (2 * a.Tq);
  const int kvh = head / a.grp;
  const int ch_half = tile < a.Tq ? 0 : 1;
  const int row0 = ch_half * a.zz.C + (tile - ch_half * a.Tq) * 128;
  const int nvalid = min(128, (ch_half + 1) * a.zz.C - row0);
  if (nvalid <= 0) return;
  const int pos0 = a.zz.pos(row0);
  const int n_kt = (pos0 + nvalid - 1) / kBwdKey + 1;
  const int wrow0 = wave * 32;
  const bool active = wrow0 < nvalid;
  const bool my_valid = wrow0 + l32 < nvalid;
  const int qpos = pos0 + min(wrow0 + l32, nvalid - 1);
  const int64_t qrow = row0 + wrow0 + l32;
  const int64_t rs = (int64_t)a.H * DH, kvs = (int64_t)a.Hkv * DH;
  const bf16 *kg = reinterpret_cast<const bf16 *>(a.k) + kvh * DH;
  const bf16 *vg = reinterpret_cast<const bf16 *>(a.v) + kvh * DH;

  bf16x8 qf[NK], df[NK];
  {
    const bf16 *qg = reinterpret_cast<const bf16 *>(a.q) + qrow * rs + head * DH;
    const bf16 *dg = reinterpret_cast<const bf16 *>(a.dout) + qrow * rs + head * DH;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      if (my_valid) {
        qf[kk] = *reinterpret_cast<const bf16x8 *>(qg + kk * 16 + g * 8);
        df[kk] = *reinterpret_cast<const bf16x8 *>(dg + kk * 16 + g * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[kk][e] = df[kk][e] = (bf16)0.f;
      }
    }
  }
  // raw products of the 64 keys of a tile held by this lane: acc[kb][v] is
  // key k0 + kb*32 + 8*(v/4) + 4*g + v%4
  auto scores = [&](const unsigned char *Ks, const bf16x8 (&bf)[NK], f32x16 (&acc)[2]) {
    const f32x16 zero = {};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(Ks, fo.row[kk] + kb * 32 * G::ROWB), bf[kk],
                                                          kk == 0 ? zero : acc[kb], 0, 0, 0);
  };
  // keys past the lane's query get -inf; only tiles that reach past the
  // wave's first query need it (c > 0, so -inf stays -inf after scaling)
  const int wmin = pos0 + wrow0;
  auto mask = [&](f32x16 (&acc)[2], int k0) {
    if (k0 + kBwdKey - 1 <= wmin) return;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = k0 + kb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
        if (key > qpos) acc[kb][v] = -INFINITY;
      }
  };

  TileRegs<DH, kBwdKey> kr, vr;
  float lse, dlt;
  {
    // ---- walk 1: row max, sum and Delta (log2 domain)
    float m = -INFINITY, l = 0.f, dsum = 0.f;
    load_tile_buf<DH, kBwdKey>(kr, kg, (int)kvs, (int)min<int64_t>(kBwdKey, a.S));
    load_tile_buf<DH, kBwdKey>(vr, vg, (int)kvs, (int)min<int64_t>(kBwdKey, a.S));
    for (int kt = 0; kt < n_kt; ++kt) {
      const int k0 = kt * kBwdKey;
      __syncthreads();
      store_tile<DH, kBwdKey>(smem[0], kr);
      store_tile<DH, kBwdKey>(smem[1], vr);
      __syncthreads();
      if (kt + 1 < n_kt) {  // next tile on its way during this one's math
        load_tile_buf<DH, kBwdKey>(kr, kg + (int64_t)(k0 + kBwdKey) * kvs, (int)kvs,
                                    (int)min<int64_t>(kBwdKey, a.S - (k0 + kBwdKey)));
        load_tile_buf<DH, kBwdKey>(vr, vg + (int64_t)(k0 + kBwdKey) * kvs, (int)kvs,
                                    (int)min<int64_t>(kBwdKey, a.S - (k0 + kBwdKey)));
      }
      if (!active) continue;
      f32x16 sacc[2], pacc[2];
      scores(smem[0], qf, sacc);
      scores(smem[1], df, pacc);
      mask(sacc, k0);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
      mx = halves_max(mx) * a.c;
      const float m_new = fmaxf(m, mx);  // finite from the first tile on (key 0 is visible)
      float part = 0.f, dpart = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v], a.c, -m_new));
          part += e;
          dpart = fmaf(e, pacc[kb][v], dpart);
        }
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l = l * alpha + part;
      dsum = dsum * alpha + dpart;
      m = m_new;
    }
    l = halves_sum(l);
    dsum = halves_sum(dsum);
    lse = m + __log2f(l);
    dlt = dsum / l;
    if (my_valid && g == 0) {
      a.lse[(int64_t)head * a.n + qrow] = lse;
      a.delta[(int64_t)head * a.n + qrow] = dlt;
    }
  }

  // ---- walk 2: dQ^T += K^T dS^T
  f32x16 qacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) qacc[db][v] = 0.f;
  load_tile_buf<DH, kBwdKey>(kr, kg, (int)kvs, (int)min<int64_t>(kBwdKey, a.S));
  load_tile_buf<DH, kBwdKey>(vr, vg, (int)kvs, (int)min<int64_t>(kBwdKey, a.S));
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * kBwdKey;
    __syncthreads();
    store_tile<DH, kBwdKey>(smem[0], kr);
    store_tile<DH, kBwdKey>(smem[1], vr);
    __syncthreads();
    if (kt + 1 < n_kt) {
      load_tile_buf<DH, kBwdKey>(kr, kg + (int64_t)(k0 + kBwdKey) * kvs, (int)kvs,
                                    (int)min<int64_t>(kBwdKey, a.S - (k0 + kBwdKey)));
      load_tile_buf<DH, kBwdKey>(vr, vg + (int64_t)(k0 + kBwdKey) * kvs, (int)kvs,
                                    (int)min<int64_t>(kBwdKey, a.S - (k0 + kBwdKey)));
    }
    if (!active) continue;
    f32x16 sacc[2], pacc[2];
    scores(smem[0], qf, sacc);
    scores(smem[1], df, pacc);  // dP^T = V dO^T
    mask(sacc, k0);
    bf16x8 ds[4], dsl[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const int kb = kq >> 1, v0 = (kq & 1) * 8;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v0 + e], a.c, -lse));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v0 + e + 1], a.c, -lse));
        put_split2<SPLIT>(ds[kq], dsl[kq], e, p0 * (pacc[kb][v0 + e] - dlt), p1 * (pacc[kb][v0 + e + 1] - dlt));
      }
    }
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16x8 kt_frag = tr_frag<DH>(smem[0], fo, db, kq);
        qacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt_frag, ds[kq], qacc[db], 0, 0, 0);
        if constexpr (SPLIT) qacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt_frag, dsl[kq], qacc[db], 0, 0, 0);
      }
  }
  // qacc[db][v] is dQ[query][32*db + 8*(v/4) + 4*g + v%4] / scale
  if (my_valid) {
    float *dq = a.dq + qrow * rs + head * DH + g * 4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq)
        *reinterpret_cast<float4 *>(dq + db * 32 + vq * 8) =
            make_float4(qacc[db][vq * 4] * a.scale, qacc[db][vq * 4 + 1] * a.scale, qacc[db][vq * 4 + 2] * a.scale,
                        qacc[db][vq * 4 + 3] * a.scale);
  }
#endif
}

// ---------------------------------------------------------------- dQ from the forward's statistics (bf16)
// The dQ walk with the forward attention's staging: K and V tiles go from
// HBM straight into LDS (buffer_load ... lds, no registers on the way),
// double-buffered, one block barrier per tile, and block (head, p) takes
// query tile T-1-p of the second chunk and then tile p of the first, so that
// every block carries the same causal work. K is stored once, in the row
// layout: the score products read its rows, and the dQ product reads it
// transposed from the same copy.
#if defined(__HIP_DEVICE_COMPILE__)
#define TSP_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))
#endif

template <int DH, bool SPLIT>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_lds_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using G = BTile<DH>;
  constexpr int ND = DH / 32, NK = DH / 16;
  constexpr int TB = kBwdKey * G::ROWB;          // one tile: 16 KB (DH 128) or 8 KB (DH 64)
  constexpr int RPW = 1024 / G::ROWB;            // rows of a 1 KB copy window
  constexpr int WPW = TB / 1024 / 4;             // copy windows per wave and tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2][TB];  // [stage][K | V]
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const FragOff<DH> fo = frag_off<DH>(lane);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head = L / a.Tq, p = L - head * a.Tq;
  const int kvh = head / a.grp;
  const int64_t rs = (int64_t)a.H * DH, kvs = (int64_t)a.Hkv * DH;
  const bf16 *kg = reinterpret_cast<const bf16 *>(a.k) + kvh * DH;
  const bf16 *vg = reinterpret_cast<const bf16 *>(a.v) + kvh * DH;

  // copy plan: window w of a tile is rows RPW*w..; the lane at row r, chunk
  // position pos loads the logical chunk that the row layout puts there
  int c_off[WPW];
#pragma unroll
  for (int i = 0; i < WPW; ++i) {
    const int row = (wave * WPW + i) * RPW + lane / G::CPR, pos = lane % G::CPR;
    c_off[i] = (int)(row * kvs * 2) + G::row_swz(row, pos) * 16;
  }
  auto copy_tile = [&](int kt, int st) {
    const int64_t k0 = (int64_t)kt * kBwdKey;
    const int rows = (int)min<int64_t>(kBwdKey, a.S - k0);
    const auto kr = __builtin_amdgcn_make_buffer_rsrc((void *)(kg + k0 * kvs), (short)0, (int)(rows * kvs * 2),
                                                      0x00020000);
    const auto vr = __builtin_amdgcn_make_buffer_rsrc((void *)(vg + k0 * kvs), (short)0, (int)(rows * kvs * 2),
                                                      0x00020000);
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const int win = wave * WPW + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, TSP_LDS_PTR(&smem[st][0][win * 1024]), 16, c_off[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, TSP_LDS_PTR(&smem[st][1][win * 1024]), 16, c_off[i], 0, 0, 0);
    }
  };
  for (int half = 0; half < 2; ++half) {
    const int ch_half = half == 0 ? 1 : 0;
    const int tile = half == 0 ? a.Tq - 1 - p : p;
    const int row0 = ch_half * a.zz.C + tile * 128;
    const int nvalid = min(128, (ch_half + 1) * a.zz.C - row0);
    if (nvalid <= 0) continue;  // the same for the whole block
    const int pos0 = a.zz.pos(row0);
    const int n_kt = (pos0 + nvalid - 1) / kBwdKey + 1;
    const int wrow0 = wave * 32;
    const bool my_valid = wrow0 + l32 < nvalid;
    const int qpos = pos0 + min(wrow0 + l32, nvalid - 1);
    const int wmin = pos0 + wrow0;
    const int64_t qrow = row0 + wrow0 + l32;

    copy_tile(0, 0);
    bf16x8 qf[NK], df[NK];
    {
      const bf16 *qp = reinterpret_cast<const bf16 *>(a.q) + qrow * rs + head * DH;
      const bf16 *dp = reinterpret_cast<const bf16 *>(a.dout) + qrow * rs + head * DH;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        bf16x8 qv = {}, dv = {};
        if (my_valid) {
          qv = *reinterpret_cast<const bf16x8 *>(qp + kk * 16 + g * 8);
          dv = *reinterpret_cast<const bf16x8 *>(dp + kk * 16 + g * 8);
        }
        qf[kk] = qv;
        df[kk] = dv;
      }
    }
    const float lse = my_valid ? a.lse[(int64_t)head * a.n + qrow] : 0.f;
    const float dlt = my_valid ? a.delta[(int64_t)head * a.n + qrow] : 0.f;
    f32x16 qacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) qacc[db][v] = 0.f;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    // key tile kt in stage st: copy tile kt + 1 into the other stage, form
    // dS from S^T = K Q^T and dP^T = V dO^T, add K^T dS^T into dQ^T; then
    // wait for this wave's copies and for every wave to be done with st
    auto step = [&](int kt, int st) {
      if (kt + 1 < n_kt) copy_tile(kt + 1, st ^ 1);
      const int k0 = kt * kBwdKey;
      const unsigned char *Ks = smem[st][0], *Vs = smem[st][1];
      const f32x16 zero = {};
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(Ks, fo.row[kk] + kb * 32 * G::ROWB), qf[kk],
                                                             kk == 0 ? zero : sacc[kb], 0, 0, 0);
          pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(Vs, fo.row[kk] + kb * 32 * G::ROWB), df[kk],
                                                             kk == 0 ? zero : pacc[kb], 0, 0, 0);
        }
      if (k0 + kBwdKey - 1 > wmin) {  // keys past the lane's query get -inf
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + kb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
            if (key > qpos) sacc[kb][v] = -INFINITY;
          }
      }
      bf16x8 ds[4], dsl[4];
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int kb = kq >> 1, v0 = (kq & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v0 + e], a.c, -lse));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v0 + e + 1], a.c, -lse));
          put_split2<SPLIT>(ds[kq], dsl[kq], e, p0 * (pacc[kb][v0 + e] - dlt), p1 * (pacc[kb][v0 + e + 1] - dlt));
        }
      }
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const bf16x8 kt_f = tr_frag<DH>(Ks, fo, db, kq);
          qacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt_f, ds[kq], qacc[db], 0, 0, 0);
          if constexpr (SPLIT) qacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt_f, dsl[kq], qacc[db], 0, 0, 0);
        }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    };
    int kt = 0;
    for (; kt + 1 < n_kt; kt += 2) {
      step(kt, 0);
      step(kt + 1, 1);
    }
    if (kt < n_kt) step(kt, 0);

    // qacc[db][v] is dQ[query][32*db + 8*(v/4) + 4*g + v%4] / scale
    if (my_valid) {
      float *dq = a.dq + qrow * rs + head * DH + g * 4;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq)
          *reinterpret_cast<float4 *>(dq + db * 32 + vq * 8) =
              make_float4(qacc[db][vq * 4] * a.scale, qacc[db][vq * 4 + 1] * a.scale, qacc[db][vq * 4 + 2] * a.scale,
                          qacc[db][vq * 4 + 3] * a.scale);
    }
  }
#endif
}

// ---------------------------------------------------------------- dK, dV (bf16)
constexpr int kBwdQ = 32;  // query rows per step of the dK/dV walk

template <int DH, bool SPLIT>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using G = BTile<DH>;
  constexpr int ND = DH / 32, NK = DH / 16;
  constexpr int TB = kBwdQ * G::ROWB;
  // Query rows are staged 64 at a time (two steps per pair of block
  // barriers; one step per pair measured 3-4% slower at 7B) into two
  // buffers that alternate: Q and dO in the row layout, and the rows'
  // statistics and positions.
  constexpr int kStage = 2 * kBwdQ;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2][2 * TB];
  // read as float4 / int4 below, so 16-byte alignment is part of the layout
  __shared__ __attribute__((aligned(16))) float lse_s[2][kStage];
  __shared__ __attribute__((aligned(16))) float dlt_s[2][kStage];
  __shared__ __attribute__((aligned(16))) int pos_s[2][kStage];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const FragOff<DH> fo = frag_off<DH>(lane);
  // the key blocks of one K/V head run on one XCD, in key order, so that
  // the blocks that run together walk nearby query rows through its L2
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kvh = L / a.Tk;
  const int64_t kb0 = (int64_t)(L % a.Tk) * 128;
  const int64_t key = kb0 + wave * 32 + l32;
  const int64_t rs = (int64_t)a.H * DH, kvs = (int64_t)a.Hkv * DH;

  bf16x8 kf[NK], vf[NK];
  {
    const bf16 *kg = reinterpret_cast<const bf16 *>(a.k) + key * kvs + kvh * DH;
    const bf16 *vg = reinterpret_cast<const bf16 *>(a.v) + key * kvs + kvh * DH;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      if (key < a.S) {
        kf[kk] = *reinterpret_cast<const bf16x8 *>(kg + kk * 16 + g * 8);
        vf[kk] = *reinterpret_cast<const bf16x8 *>(vg + kk * 16 + g * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[kk][e] = vf[kk][e] = (bf16)0.f;
      }
    }
  }
  f32x16 kacc[ND], vacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) kacc[db][v] = vacc[db][v] = 0.f;
  const int wkey0 = (int)kb0 + wave * 32;  // first key of this wave

  // S = Q K^T and dP = dO V^T of the step in buffer b, keys on the lanes:
  // one MFMA chain each, started from a zero constant; the two chains
  // interleave with each other and with the previous step's update (the
  // chains split into even and odd K slices measured 2% slower: their
  // merge costs 32 additions and, with the accumulators in AGPRs, 64 reads
  // back per step)
  auto scores = [&](int b, int sub, f32x16 &sacc, f32x16 &pacc) {
    const f32x16 zero = {};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(smem[b][0] + sub * TB, fo.row[kk]), kf[kk],
                                                     kk == 0 ? zero : sacc, 0, 0, 0);
      pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(smem[b][1] + sub * TB, fo.row[kk]), vf[kk],
                                                     kk == 0 ? zero : pacc, 0, 0, 0);
    }
  };
  // sacc[v]: S[row 8*(v/4) + 4*g + v%4][key]. P and dS of the step in buffer
  // b in the B-operand order (rows past the chunk carry position -1, so the
  // masked form zeroes them), then dV^T += dO^T P and dK^T += Q^T dS.
  auto update = [&](auto masked, int b, int sub, const f32x16 &sacc, const f32x16 &pacc) {
    bf16x8 ph[2], dh[2], p_lo[2], ds_lo[2];
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
      const int r = sub * kBwdQ + m4 * 8 + g * 4;
      const float4 ls = *reinterpret_cast<const float4 *>(&lse_s[b][r]);
      const float4 dl = *reinterpret_cast<const float4 *>(&dlt_s[b][r]);
      const float lsv[4] = {ls.x, ls.y, ls.z, ls.w}, dlv[4] = {dl.x, dl.y, dl.z, dl.w};
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[m4 * 4 + e], a.c, -lsv[e]));
      if constexpr (decltype(masked)::value) {
        const int4 ps = *reinterpret_cast<const int4 *>(&pos_s[b][r]);
        const int psv[4] = {ps.x, ps.y, ps.z, ps.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (key > psv[e]) pv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int v = m4 * 4 + e;  // v, v + 1 share the fragment (v is even)
        put_split2<SPLIT>(ph[v >> 3], p_lo[v >> 3], v & 7, pv[e], pv[e + 1]);
        put_split2<SPLIT>(dh[v >> 3], ds_lo[v >> 3], v & 7, pv[e] * (pacc[v] - dlv[e]),
                          pv[e + 1] * (pacc[v + 1] - dlv[e + 1]));
      }
    }
#pragma unroll
    for (int mu = 0; mu < 2; ++mu)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16x8 dot = tr_frag<DH>(smem[b][1] + sub * TB, fo, db, mu);
        const bf16x8 qt = tr_frag<DH>(smem[b][0] + sub * TB, fo, db, mu);
        vacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dot, ph[mu], vacc[db], 0, 0, 0);
        kacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, dh[mu], kacc[db], 0, 0, 0);
        if constexpr (SPLIT) {
          vacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dot, p_lo[mu], vacc[db], 0, 0, 0);
          kacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, ds_lo[mu], kacc[db], 0, 0, 0);
        }
      }
  };

  for (int hi = 0; hi < a.grp; ++hi) {
    const int head = kvh * a.grp + hi;
    const bf16 *qg = reinterpret_cast<const bf16 *>(a.q) + head * DH;
    const bf16 *dg = reinterpret_cast<const bf16 *>(a.dout) + head * DH;
    for (int chh = 0; chh < 2; ++chh) {
      const int base = chh == 0 ? a.zz.base0 : a.zz.base1;  // position of the chunk's first row
      const int t_end = (chh + 1) * a.zz.C;
      const int t_lo = chh * a.zz.C + (int)max<int64_t>(0, kb0 - base);  // first row that sees a key of the block
      if (t_lo >= t_end) continue;
      TileRegs<DH, kStage> qr, dr;
      float st_lse = 0.f, st_dlt = 0.f;
      auto fetch = [&](int t0) {  // a stage's rows into registers (statistics: threads < kStage)
        const int nv = min(kStage, t_end - t0);
        load_tile_buf<DH, kStage>(qr, qg + (int64_t)t0 * rs, (int)rs, nv);
        load_tile_buf<DH, kStage>(dr, dg + (int64_t)t0 * rs, (int)rs, nv);
        const auto lr = __builtin_amdgcn_make_buffer_rsrc((void *)(a.lse + (int64_t)head * a.n + t0), (short)0,
                                                          nv * 4, 0x00020000);
        const auto dr_ = __builtin_amdgcn_make_buffer_rsrc((void *)(a.delta + (int64_t)head * a.n + t0), (short)0,
                                                           nv * 4, 0x00020000);
        st_lse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lr, (int)threadIdx.x * 4, 0, 0));
        st_dlt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dr_, (int)threadIdx.x * 4, 0, 0));
      };
      auto stage = [&](int b, int t0) {  // the fetched rows into buffer b
        store_tile<DH, kStage>(smem[b][0], qr);
        store_tile<DH, kStage>(smem[b][1], dr);
        if (threadIdx.x < kStage) {
          const int t = t0 + threadIdx.x;
          const bool ok = t < t_end;
          lse_s[b][threadIdx.x] = ok ? st_lse : 0.f;
          dlt_s[b][threadIdx.x] = ok ? st_dlt : 0.f;
          pos_s[b][threadIdx.x] = ok ? base + (t - chh * a.zz.C) : -1;
        }
      };
      // Rows past the chunk, or before some key of the wave, need the mask;
      // the rest of the walk does not. A step whose rows all lie before the
      // wave's keys runs masked (all its probabilities are zero).
      auto need_mask = [&](int t0) {
        return t0 + kBwdQ > t_end || base + (t0 - chh * a.zz.C) < wkey0 + 31;
      };
      // Software pipeline over the walk's steps: step i's scores are taken
      // one iteration ahead, while step i-1's probabilities and products are
      // formed, so that the exponentials and conversions issue under the
      // score MFMAs of the next step. The stage after next is fetched into
      // registers while the current one is in use.
      fetch(t_lo);
      __syncthreads();  // the previous walk's reads of both buffers are done
      stage(0, t_lo);
      __syncthreads();
      if (t_lo + kStage < t_end) fetch(t_lo + kStage);
      f32x16 s0, p0, s1, p1;
      scores(0, 0, s0, p0);
      // issue order of the block: each of the 16 score MFMAs followed by
      // four VALU instructions of the update (five with P and dS split,
      // whose update has three conversions per value), so that the update's
      // exponentials and conversions run while the matrix core works (with
      // 64-row stages, three, five and six measured slower for plain P and
      // dS; four cost the split form 4%)
      auto interleave = [] {
#pragma unroll
        for (int i = 0; i < 2 * NK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, SPLIT ? 5 : 4, 0);
        }
      };
      // One pipeline iteration: score the next step and finish step t0,
      // which sits in half `sub` of buffer b; the next step is the other
      // half of b (sub 0) or the first half of b ^ 1, staged here (sub 1).
      // Returns false after the last step. The scores and the update share
      // one basic block, so that the scheduler can interleave them (after
      // the last step the scores read a stale buffer and are dropped).
      auto iter = [&](int b, int sub, int t0, f32x16 &sc, f32x16 &pc, f32x16 &sn, f32x16 &pn) {
        const bool next = t0 + kBwdQ < t_end;
        const int nb = sub ? b ^ 1 : b, nsub = sub ^ 1;
        if (sub && next) {
          __syncthreads();  // every wave is done with buffer b ^ 1
          stage(b ^ 1, t0 + kBwdQ);
          __syncthreads();
          if (t0 + kBwdQ + kStage < t_end) fetch(t0 + kBwdQ + kStage);
        }
        if (need_mask(t0)) {
          scores(nb, nsub, sn, pn);
          update(std::true_type{}, b, sub, sc, pc);
          interleave();
        } else {
          scores(nb, nsub, sn, pn);
          update(std::false_type{}, b, sub, sc, pc);
          interleave();
        }
        return next;
      };
      for (int t0 = t_lo;; t0 += 4 * kBwdQ) {
        if (!iter(0, 0, t0, s0, p0, s1, p1)) break;
        if (!iter(0, 1, t0 + kBwdQ, s1, p1, s0, p0)) break;
        if (!iter(1, 0, t0 + 2 * kBwdQ, s0, p0, s1, p1)) break;
        if (!iter(1, 1, t0 + 3 * kBwdQ, s1, p1, s0, p0)) break;
      }
    }
  }
  // kacc/vacc[db][v]: feature 32*db + 8*(v/4) + 4*g + v%4 of this lane's key
  if (key < a.S) {
    float *dk = a.dk + key * kvs + kvh * DH + g * 4;
    float *dv = a.dv + key * kvs + kvh * DH + g * 4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        *reinterpret_cast<float4 *>(dk + db * 32 + vq * 8) =
            make_float4(kacc[db][vq * 4] * a.dk_scale, kacc[db][vq * 4 + 1] * a.dk_scale,
                        kacc[db][vq * 4 + 2] * a.dk_scale, kacc[db][vq * 4 + 3] * a.dk_scale);
        *reinterpret_cast<float4 *>(dv + db * 32 + vq * 8) =
            make_float4(vacc[db][vq * 4], vacc[db][vq * 4 + 1], vacc[db][vq * 4 + 2], vacc[db][vq * 4 + 3]);
      }
  }
#endif
}

// ---------------------------------------------------------------- fp32
// Row statistics and dQ: one thread per (query row, head), exact expf; the
// log-sum-exp is kept in the log2 domain like the bf16 path.
template <int DH>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(BwdArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int head = blockIdx.y;
  if (row >= a.n) return;
  const int qpos = a.zz.pos((int32_t)row);
  const int64_t rs = (int64_t)a.H * DH, kvs = (int64_t)a.Hkv * DH;
  const float *q = reinterpret_cast<const float *>(a.q) + row * rs + head * DH;
  const float *dout = reinterpret_cast<const float *>(a.dout) + row * rs + head * DH;
  const float *k = reinterpret_cast<const float *>(a.k) + (head / a.grp) * DH;
  const float *v = reinterpret_cast<const float *>(a.v) + (head / a.grp) * DH;
  float m = -INFINITY, l = 0.f, dsum = 0.f;
  for (int u = 0; u <= qpos; ++u) {
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < DH; ++d) {
      s = fmaf(q[d], k[(int64_t)u * kvs + d], s);
      dp = fmaf(dout[d], v[(int64_t)u * kvs + d], dp);
    }
    s *= a.scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new), e = expf(s - m_new);
    l = l * alpha + e;
    dsum = dsum * alpha + e * dp;
    m = m_new;
  }
  const float lse_nat = m + logf(l);
  const float dlt = dsum / l;
  a.lse[(int64_t)head * a.n + row] = lse_nat * 1.4426950408889634f;
  a.delta[(int64_t)head * a.n + row] = dlt;
  float acc[DH];
  for (int d = 0; d < DH; ++d) acc[d] = 0.f;
  for (int u = 0; u <= qpos; ++u) {
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < DH; ++d) {
      s = fmaf(q[d], k[(int64_t)u * kvs + d], s);
      dp = fmaf(dout[d], v[(int64_t)u * kvs + d], dp);
    }
    const float ds = expf(s * a.scale - lse_nat) * (dp - dlt);
    for (int d = 0; d < DH; ++d) acc[d] = fmaf(ds, k[(int64_t)u * kvs + d], acc[d]);
  }
  float *dq = a.dq + row * rs + head * DH;
  for (int d = 0; d < DH; ++d) dq[d] = acc[d] * a.scale;
}

// dK, dV: one thread per (key, K/V head) over every query row that sees the
// key, in every query head of the group.
template <int DH>
__global__ __launch_bounds__(64) void attn_bwd_dkv_f32_kernel(BwdArgs a) {
  const int64_t key = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int kvh = blockIdx.y;
  if (key >= a.S) return;
  const int64_t rs = (int64_t)a.H * DH, kvs = (int64_t)a.Hkv * DH;
  const float *k = reinterpret_cast<const float *>(a.k) + key * kvs + kvh * DH;
  const float *v = reinterpret_cast<const float *>(a.v) + key * kvs + kvh * DH;
  float gk[DH], gv[DH];
  for (int d = 0; d < DH; ++d) gk[d] = gv[d] = 0.f;
  for (int hi = 0; hi < a.grp; ++hi) {
    const int head = kvh * a.grp + hi;
    for (int t = 0; t < a.n; ++t) {
      if (a.zz.pos(t) < key) continue;
      const float *q = reinterpret_cast<const float *>(a.q) + (int64_t)t * rs + head * DH;
      const float *dout = reinterpret_cast<const float *>(a.dout) + (int64_t)t * rs + head * DH;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < DH; ++d) {
        s = fmaf(q[d], k[d], s);
        dp = fmaf(dout[d], v[d], dp);
      }
      const float lse_nat = a.lse[(int64_t)head * a.n + t] * 0.69314718055994531f;
      const float p = expf(s * a.scale - lse_nat);
      const float ds = p * (dp - a.delta[(int64_t)head * a.n + t]);
      for (int d = 0; d < DH; ++d) {
        gk[d] = fmaf(ds, q[d], gk[d]);
        gv[d] = fmaf(p, dout[d], gv[d]);
      }
    }
  }
  float *dk = a.dk + key * kvs + kvh * DH;
  float *dv = a.dv + key * kvs + kvh * DH;
  for (int d = 0; d < DH; ++d) {
    dk[d] = gk[d] * a.scale;
    dv[d] = gv[d];
  }
}

hipError_t launch_attention_bwd(int dtype, const void *q, const void *k, const void *v, const void *dout, float *dq,
                                float *dk, float *dv, float *lse, float *delta, int64_t S, int32_t n, int32_t H,
                                int32_t Hkv, int32_t Dh, float scale, ZigzagMap zz, hipStream_t s,
                                const float *o_f32, const float *lse_in, bool split, bool q_prescaled) {
  if (n <= 0) return hipSuccess;
  if (Hkv < 1 || H % Hkv != 0 || (Dh != 64 && Dh != 128)) return hipErrorInvalidValue;
  const bool given = o_f32 != nullptr && lse_in != nullptr;
  if (given && dtype != TSP_BF16) return hipErrorInvalidValue;
  if (q_prescaled && !given) return hipErrorInvalidValue;
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.o_f32 = o_f32;
  a.lse_in = lse_in;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.lse = lse;
  a.delta = delta;
  a.S = S;
  a.n = n;
  a.H = H;
  a.Hkv = Hkv;
  a.grp = H / Hkv;
  a.scale = scale;
  // multiplier of the scores in the exp2 domain, kept at least the smallest
  // normal float so that masked scores (-inf) stay -inf with a zero scale
  a.c = fmaxf(scale * 1.4426950408889634f, 1.17549435e-38f);
  a.dk_scale = scale;
  if (q_prescaled) {  // the scores come out of the products in the log2 domain
    a.c = 1.0f;
    a.dk_scale = 0.69314718055994531f;
  }
  a.zz = zz;
  a.Tq = (zz.C + 127) / 128;
  a.Tk = (int32_t)((S + 127) / 128);
  if (dtype == TSP_BF16) {
    const dim3 qgrid(H * 2 * a.Tq), kgrid(Hkv * a.Tk);
    if (given) {  // statistics from the forward, then dQ without its first walk
      const int64_t rows = (int64_t)n * H;
      hipLaunchKernelGGL(attn_bwd_stats_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, a, (int)Dh);
    }
    // one instantiation per (head width, statistics given, P/dS split)
    auto launch = [&](auto dh, auto gv, auto sp) {
      constexpr int DH = decltype(dh)::value;
      constexpr bool GV = decltype(gv)::value, SP = decltype(sp)::value;
      if constexpr (GV)  // paired query tiles: one block per (head, tile pair)
        hipLaunchKernelGGL((attn_bwd_dq_lds_kernel<DH, SP>), dim3(H * a.Tq), dim3(256), 0, s, a);
      else  // statistics walk, then dQ
        hipLaunchKernelGGL((attn_bwd_dq_kernel<DH, SP>), qgrid, dim3(256), 0, s, a);
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<DH, SP>), kgrid, dim3(256), 0, s, a);
    };
    using I128 = std::integral_constant<int, 128>;
    using I64 = std::integral_constant<int, 64>;
    using T = std::true_type;
    using F = std::false_type;
    if (Dh == 128) {
      if (given)
        split ? launch(I128{}, T{}, T{}) : launch(I128{}, T{}, F{});
      else
        split ? launch(I128{}, F{}, T{}) : launch(I128{}, F{}, F{});
    } else {
      if (given)
        split ? launch(I64{}, T{}, T{}) : launch(I64{}, T{}, F{});
      else
        split ? launch(I64{}, F{}, T{}) : launch(I64{}, F{}, F{});
    }
  } else {
    const dim3 qgrid((n + 63) / 64, H), kgrid((unsigned)((S + 63) / 64), Hkv);
    if (Dh == 128) {
      hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<128>, qgrid, dim3(64), 0, s, a);
      hipLaunchKernelGGL(attn_bwd_dkv_f32_kernel<128>, kgrid, dim3(64), 0, s, a);
    } else {
      hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<64>, qgrid, dim3(64), 0, s, a);
      hipLaunchKernelGGL(attn_bwd_dkv_f32_kernel<64>, kgrid, dim3(64), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace tsp
