// Causal attention of one rank's zigzag-ordered queries against the gathered
// full-sequence K/V, on the gfx950 matrix cores.
//
// Work split: the rank's local rows form two chunks (global positions r*C..
// and (2D-1-r)*C..). They are cut into T = ceil(C/128) query tiles per chunk;
// block (head, p) takes the mirrored tile T-1-p of the second chunk and then
// tile p of the first, so every block walks about S/64 + 2 key tiles and all
// blocks carry equal causal work. The long (second-chunk) tile goes first: the
// blocks of one head run together on one XCD and stream the same key tiles
// through its L2 (at 7B the L2's requests to memory come to about twice the
// K/V bytes, as the blocks drift apart and the short walks restart from key
// 0). Key tiles past a tile's last query are never loaded; only tiles that
// straddle the diagonal apply the mask.
//
// Per block: 4 waves x 32 queries, two blocks per CU. K and V tiles of 64 keys
// go from HBM straight into LDS (buffer_load ... lds, 16 bytes per lane, no
// registers on the way), two stages deep: the next tile's copy is issued
// before the current tile's math. Both stay row-major in LDS with their
// 16-byte chunks XOR-swizzled by row (the copying lane picks the source
// chunk), so every fragment read below is free of bank conflicts.
//
// Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K rows read
// with ds_read_b128), so a lane owns one query and 32 of the tile's keys.
// Softmax runs in the exp2 domain against a per-row reference max m that is
// taken on the walk's first key tile and raised only on the rare tile whose
// probabilities would grow too large; the S^T accumulators start at -m, so
// with Q pre-multiplied by scale * log2(e) (the layer's QKV epilogue stores it
// that way) a probability is one exp2 of an accumulator, and otherwise one
// multiply and an exp2. No per-tile row max is needed: a tile is accepted
// when each lane's sum of its probabilities stays below a fixed bound, which
// also bounds every probability; otherwise the tile is redone with m raised
// to its max and O and l rescaled. P is rounded to bf16 (v_cvt_pk_bf16_f32)
// and summed from the rounded values (v_dot2c_f32_bf16). O^T = V^T P^T runs on
// the same MFMA with P taken straight from the score registers; its V^T
// operand comes from two ds_read_b64_tr_b16 per lane, each a 4x4 transpose of
// 16-bit elements inside 16 lanes, which hands every lane 4 consecutive keys
// of one feature in the key order the score registers have.
//
// Query tiles whose positions all lie below kSplitPos see so few keys that one
// probability can carry most of a row; there P is applied as a bf16 pair
// hi + lo (two MFMAs), which keeps the product accurate to about 2^-16 of |P|.
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
  int32_t Hkv, grp;  // K/V heads; query head i reads K/V head i / grp, grp = H / Hkv
  float scale;  // softmax scale
  float c;      // scale * log2(e)
  ZigzagMap zz;
  int32_t T;         // query tiles per chunk
  int64_t o_panel;   // bf16 O: panel stride (64-column panels) or 0 for [n][H][Dh]
  float *lse;        // [H][n] natural log-sum-exp of each row's scaled scores (LSE variant only)
};

constexpr int kBQ = 128, kBKey = 64, kAttnThreads = 256;
// Query tiles whose last position is below this use the hi + lo split of P.
[[maybe_unused]] constexpr int kSplitPos = 1024;

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define TSP_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Geometry of one K or V tile (64 rows of DH bf16) in LDS.
template <int DH>
struct KvTile {
  static constexpr int ROWB = DH * 2;                     // bytes per row
  static constexpr int CPR = DH / 8;                      // 16-byte chunks per row
  static constexpr int BYTES = kBKey * ROWB;              // 16 KB (DH 128) or 8 KB (DH 64)
  static constexpr int ROWS_PER_KB = 1024 / ROWB;         // rows per 1 KB copy window
  static constexpr int WIN_PER_WAVE = BYTES / 1024 / 4;   // copy windows per wave
  // Chunk position of logical chunk ch of a K row: the 16 rows that one
  // 16-lane group reads (same logical chunk) land in 16 distinct bank groups.
  static __device__ __forceinline__ int k_swz(int row, int ch) {
    return ch ^ (CPR == 16 ? (row & 15) : ((row >> 1) & 7));
  }
  // Chunk position of logical chunk ch of a V row: the 4 rows x 4 chunks that
  // one transpose read of 32 lanes touches land in 16 distinct bank groups.
  static __device__ __forceinline__ int v_swz(int row, int ch) {
    return ch ^ (CPR == 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1));
  }
};

// The descriptor type and the LDS-copy builtins exist only for the device
// target, so the helpers and the kernel body below are compiled in the device
// pass only (the host pass just needs the kernel's signature for its stub).
#if defined(__HIP_DEVICE_COMPILE__)
// Buffer descriptor over rows [k0, min(k0 + 64, S)) of one head of K or V:
// loads past the last valid row return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16 *head_base, int64_t k0, int64_t S,
                                                            int64_t rs) {
  const int64_t rows = min<int64_t>(kBKey, S - k0);
  return __builtin_amdgcn_make_buffer_rsrc((void *)(head_base + k0 * rs), (short)0, (int)(rows * rs * 2),
                                           0x00020000);
}

// One 64-key tile for one wave: scores, online softmax, O^T += V^T P^T.
// MASK: the tile reaches past some query of the wave (diagonal tile).
// SPLIT: P enters the product as bf16 hi + lo.
// Lane-constant LDS byte offsets of the fragment reads, relative to a tile:
// k[kk]: the 16-byte K chunk (row lane%32, logical chunk 2*kk + lane/32);
// rows 32.. of the tile are a constant 32*ROWB further (same swizzle).
// v[db]: the transpose-read address for 32-feature block db and key group 0;
// key group kq, half hv adds the constant (16*kq + 8*hv)*ROWB (the swizzle
// depends only on key % 4, which those offsets keep).
template <int DH>
struct FragAddr {
  int k[DH / 16];
  int v[DH / 32];
};

template <int DH>
__device__ __forceinline__ FragAddr<DH> frag_addr(int lane) {
  using G = KvTile<DH>;
  FragAddr<DH> fa;
  const int g = lane >> 5, l32 = lane & 31, r16 = lane & 15, dsub = (lane >> 4) & 1;
#pragma unroll
  for (int kk = 0; kk < DH / 16; ++kk) fa.k[kk] = l32 * G::ROWB + G::k_swz(l32, kk * 2 + g) * 16;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db) {
    const int key = g * 4 + (r16 >> 2);
    const int dstart = db * 32 + dsub * 16 + 4 * (r16 & 3);
    fa.v[db] = key * G::ROWB + G::v_swz(key, dstart >> 3) * 16 + (dstart & 7) * 2;
  }
  return fa;
}

// Probabilities of the 64 scores held by the lane, minus a shift (log2
// domain): P as bf16 (hi, and lo = p - hi when SPLIT) in MFMA B-operand
// order, and the lane's sum of them. Masked keys hold -inf and get 0 (the
// multiplier c is never 0: see launch_attention).
template <bool SHIFT, bool SPLIT, bool QPRE>
__device__ __forceinline__ float tile_probs(const f32x16 (&sacc)[2], float shift, float c, bf16x8 (&ph)[4],
                                            bf16x8 (&pl)[4]) {
  const float nsc = -shift * c;
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  float lt = 0.f;
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
    const int kb = kq >> 1, v0 = (kq & 1) * 8;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float s0 = sacc[kb][v0 + e], s1 = sacc[kb][v0 + e + 1];
      const float x0 = QPRE ? (SHIFT ? s0 - shift : s0) : (SHIFT ? fmaf(s0, c, nsc) : s0 * c);
      const float x1 = QPRE ? (SHIFT ? s1 - shift : s1) : (SHIFT ? fmaf(s1, c, nsc) : s1 * c);
      const float p0 = __builtin_amdgcn_exp2f(x0), p1 = __builtin_amdgcn_exp2f(x1);
      const bf16x2 h2 = {(bf16)p0, (bf16)p1};
      ph[kq][e] = h2[0];
      ph[kq][e + 1] = h2[1];
      if constexpr (SPLIT) {
        const bf16x2 l2 = {(bf16)(p0 - (float)h2[0]), (bf16)(p1 - (float)h2[1])};
        pl[kq][e] = l2[0];
        pl[kq][e + 1] = l2[1];
        lt += p0 + p1;
      } else {
        lt = __builtin_amdgcn_fdot2_f32_bf16(h2, ones, lt, false);
      }
    }
  }
  return lt;
}

// Largest sum of one lane's 32 probabilities (relative to the row's
// reference max m) that a tile accepts without raising m: every probability
// of an accepted tile is at most 2^16, and O and l stay far from fp32
// overflow over any sequence length the entry points take.
constexpr float kLaneSumLimit = 65536.0f;

// One 64-key tile for one wave: scores, online softmax, O^T += V^T P^T.
// Q arrives pre-multiplied by scale * log2(e), so scores are in the log2
// domain. The accumulators of S^T start at -m (bias, one value per lane), so
// they hold s - m and the probabilities need only exp2. The reference max m
// is fixed on the walk's first tile (key 0 is in it and visible to every
// query) and raised only on a tile whose probabilities would pass
// kLaneSumLimit (or overflow); that tile is then redone from its scores.
// MASK: the tile reaches past some query of the wave (diagonal tile).
// SPLIT: P enters the product as bf16 hi + lo.
template <int DH, bool MASK, bool SPLIT, bool QPRE>
__device__ __forceinline__ void attn_tile(const unsigned char *__restrict__ Ks, const unsigned char *__restrict__ Vs,
                                          const FragAddr<DH> &fa, const bf16x8 (&qf)[DH / 16],
                                          f32x16 (&oacc)[DH / 32], f32x16 &bias, float &m_run, float &l_part,
                                          int kstart, int qpos, bool first, float c, int lane) {
  using G = KvTile<DH>;
  constexpr int ND = DH / 32;
  const int g = lane >> 5;
  // ---- S^T - m = K Q^T + bias for the 64 keys: two independent 32-key
  // accumulators (raised issue priority while this wave feeds the matrix
  // pipe, so the other wave of the SIMD fills the gaps with its softmax)
  __builtin_amdgcn_s_setprio(1);
  f32x16 sacc[2];
#pragma unroll
  for (int kk = 0; kk < DH / 16; ++kk)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + fa.k[kk] + kb * 32 * G::ROWB);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], kk == 0 ? bias : sacc[kb], 0, 0, 0);
    }
  __builtin_amdgcn_s_setprio(0);
  // sacc[kb][v] is the score of key kstart + kb*32 + 8*(v/4) + 4*g + v%4
  if constexpr (MASK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kstart + kb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
        if (key > qpos) sacc[kb][v] = -INFINITY;
      }
  }
  bf16x8 ph[4], pl[4];
  float lt = 0.f;
  bool redo = first;
  if (!first) {
    lt = tile_probs<false, SPLIT, QPRE>(sacc, 0.f, c, ph, pl);
    // !(x <= limit) also catches an overflow to inf
    redo = __any(!(lt <= kLaneSumLimit));
  }
  if (redo) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = halves_max(mx);
    // On the first tile (bias 0) mx is the row's max score, finite; later,
    // mx is -inf only when every key of the tile is masked for the query.
    const float delta = first ? mx : fmaxf(mx, 0.f);
    if (!first) {
      const float alpha = __builtin_amdgcn_exp2f(QPRE ? -delta : -delta * c);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
    }
    m_run += delta;
#pragma unroll
    for (int v = 0; v < 16; ++v) bias[v] = -m_run;
    lt = tile_probs<true, SPLIT, QPRE>(sacc, delta, c, ph, pl);
  }
  l_part += lt;
  // ---- O^T += V^T P^T, 16 keys per step
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      // transpose read: lane r of each 16-lane group points at key
      // 16*kq + 8*hv + 4*g + r/4 and features 16*((lane/16)%2) + 4*(r%4) .. +3
      // of block db; it receives 4 consecutive keys of feature r of that group
      s16x4 part[2];
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        const unsigned char *addr = Vs + fa.v[db] + (kq * 16 + hv * 8) * G::ROWB;
        part[hv] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(addr));
      }
      const s16x8_t both = {part[0][0], part[0][1], part[0][2], part[0][3],
                            part[1][0], part[1][1], part[1][2], part[1][3]};
      const bf16x8 vf = __builtin_bit_cast(bf16x8, both);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ph[kq], oacc[db], 0, 0, 0);
      if constexpr (SPLIT) oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[kq], oacc[db], 0, 0, 0);
    }
  }
}

// What one block needs to copy K/V tiles of its head into LDS.
template <int DH>
struct KvCopy {
  const bf16 *kg, *vg;  // head column of K and V
  int64_t S, rs;        // rows, row pitch (elements)
  int wave;
  int k_off[KvTile<DH>::WIN_PER_WAVE], v_off[KvTile<DH>::WIN_PER_WAVE];
};

// Copy key tile kt into LDS stage st (this wave's windows).
template <int DH>
__device__ __forceinline__ void copy_tile(const KvCopy<DH> &cp, unsigned char (*smem)[2][KvTile<DH>::BYTES], int kt,
                                          int st) {
  using G = KvTile<DH>;
  const int64_t k0 = (int64_t)kt * kBKey;
  const __amdgpu_buffer_rsrc_t kr = tile_rsrc(cp.kg, k0, cp.S, cp.rs);
  const __amdgpu_buffer_rsrc_t vr = tile_rsrc(cp.vg, k0, cp.S, cp.rs);
#pragma unroll
  for (int i = 0; i < G::WIN_PER_WAVE; ++i) {
    const int win = cp.wave * G::WIN_PER_WAVE + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, TSP_LDS(&smem[st][0][win * 1024]), 16, cp.k_off[i], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, TSP_LDS(&smem[st][1][win * 1024]), 16, cp.v_off[i], 0, 0, 0);
  }
}

// Key tiles [kt0, kt1) of a walk of n_kt tiles: the tile in stage kt & 1 is
// already in LDS when tile kt starts; tile kt + 1 is copied meanwhile. Each
// variant runs its own loop so that the hot one carries no rare-case code.
template <int DH, bool MASK, bool SPLIT, bool QPRE, int CUR>
__device__ __forceinline__ void attn_step(const KvCopy<DH> &cp, unsigned char (*smem)[2][KvTile<DH>::BYTES], int kt,
                                          int n_kt, bool active, int wmax, const FragAddr<DH> &fa,
                                          const bf16x8 (&qf)[DH / 16],
                                          f32x16 (&oacc)[DH / 32], f32x16 &bias, float &m_run, float &l_part, int qpos,
                                          float c, int lane) {
  if (kt + 1 < n_kt) copy_tile<DH>(cp, smem, kt + 1, CUR ^ 1);
  const int kstart = kt * kBKey;
  if (active && (!MASK || kstart <= wmax))
    attn_tile<DH, MASK, SPLIT, QPRE>(smem[CUR][0], smem[CUR][1], fa, qf, oacc, bias, m_run, l_part, kstart, qpos,
                                     kt == 0, c, lane);
  // the next tile's copy has landed (this wave's part), and every wave is
  // done with the current stage before it is overwritten
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
}

// Key tiles [kt0, kt1) of a walk of n_kt tiles: tile kt sits in LDS stage
// kt & 1 when it starts, and tile kt + 1 is copied meanwhile. The loop runs
// two tiles per trip so that each stage's LDS offsets are constants. Each
// variant runs its own loop so that the hot one carries no rare-case code.
template <int DH, bool MASK, bool SPLIT, bool QPRE>
__device__ __forceinline__ void attn_walk(const KvCopy<DH> &cp, unsigned char (*smem)[2][KvTile<DH>::BYTES], int kt0,
                                          int kt1, int n_kt, bool active, int wmax, const FragAddr<DH> &fa,
                                          const bf16x8 (&qf)[DH / 16],
                                          f32x16 (&oacc)[DH / 32], f32x16 &bias, float &m_run, float &l_part, int qpos,
                                          float c, int lane) {
  int kt = kt0;
  if (kt < kt1 && (kt & 1)) {
    attn_step<DH, MASK, SPLIT, QPRE, 1>(cp, smem, kt, n_kt, active, wmax, fa, qf, oacc, bias, m_run, l_part, qpos, c,
                                        lane);
    ++kt;
  }
  for (; kt + 1 < kt1; kt += 2) {
    attn_step<DH, MASK, SPLIT, QPRE, 0>(cp, smem, kt, n_kt, active, wmax, fa, qf, oacc, bias, m_run, l_part, qpos, c,
                                        lane);
    attn_step<DH, MASK, SPLIT, QPRE, 1>(cp, smem, kt + 1, n_kt, active, wmax, fa, qf, oacc, bias, m_run, l_part, qpos,
                                        c, lane);
  }
  if (kt < kt1)
    attn_step<DH, MASK, SPLIT, QPRE, 0>(cp, smem, kt, n_kt, active, wmax, fa, qf, oacc, bias, m_run, l_part, qpos, c,
                                        lane);
}
#endif  // __HIP_DEVICE_COMPILE__

template <int DH, bool OUT_F32, bool QPRE, bool LSE = false>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_bf16_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using G = KvTile<DH>;
  constexpr int ND = DH / 32;  // 32-row blocks of O^T
  // [stage][K | V][tile]
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2][G::BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head = L / a.T, p = L - (L / a.T) * a.T;
  const int64_t rs = (int64_t)a.H * DH;  // row pitch of q and o (elements)
  const int kvh = head / a.grp;
  const bf16 *qg = reinterpret_cast<const bf16 *>(a.q) + head * DH;

  // Copy windows of this wave: window w covers rows w*ROWS_PER_KB.. of the
  // tile; lane -> (row, chunk position); it loads the logical chunk that
  // belongs at that position.
  KvCopy<DH> cp;
  cp.kg = reinterpret_cast<const bf16 *>(a.k) + kvh * DH;
  cp.vg = reinterpret_cast<const bf16 *>(a.v) + kvh * DH;
  cp.S = a.S;
  cp.rs = (int64_t)a.Hkv * DH;
  cp.wave = wave;
#pragma unroll
  for (int i = 0; i < G::WIN_PER_WAVE; ++i) {
    const int win = wave * G::WIN_PER_WAVE + i;
    const int row = win * G::ROWS_PER_KB + lane / G::CPR, pos = lane % G::CPR;
    cp.k_off[i] = (int)(row * cp.rs * 2) + G::k_swz(row, pos) * 16;
    cp.v_off[i] = (int)(row * cp.rs * 2) + G::v_swz(row, pos) * 16;
  }

  const FragAddr<DH> fa = frag_addr<DH>(lane);

  for (int half = 0; half < 2; ++half) {
    const int tile = half == 0 ? 2 * a.T - 1 - p : p;
    const int ch_half = tile < a.T ? 0 : 1;
    const int row0 = ch_half * a.zz.C + (tile - ch_half * a.T) * kBQ;  // first local row of the tile
    const int nvalid = min(kBQ, (ch_half + 1) * a.zz.C - row0);
    const int pos0 = a.zz.pos(row0);  // positions are consecutive inside a tile
    const int n_kt = (pos0 + nvalid - 1) / kBKey + 1;
    // key tiles below kt_diag lie wholly at or before every query of the block
    const int kt_diag = min(n_kt, (pos0 + 1) / kBKey);
    const bool split = pos0 + nvalid - 1 < kSplitPos;

    const int wrow0 = wave * 32;
    const int w_nvalid = max(0, min(32, nvalid - wrow0));
    const int wmax = pos0 + wrow0 + w_nvalid - 1;
    const bool active = w_nvalid > 0;
    const bool my_valid = wrow0 + l32 < nvalid;
    const int qpos = pos0 + min(wrow0 + l32, nvalid - 1);
    const int64_t qrow = row0 + wrow0 + l32;

    copy_tile<DH>(cp, smem, 0, 0);

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
    // reference max (log2 domain) and the S^T accumulators' start value -m;
    // the first key tile sets both
    float m_run = 0.f, l_part = 0.f;
    f32x16 bias;
#pragma unroll
    for (int v = 0; v < 16; ++v) bias[v] = 0.f;

    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    if (split) {
      attn_walk<DH, true, true, QPRE>(cp, smem, 0, n_kt, n_kt, active, wmax, fa, qf, oacc, bias, m_run, l_part, qpos,
                                      a.c, lane);
    } else {
      attn_walk<DH, false, false, QPRE>(cp, smem, 0, kt_diag, n_kt, active, wmax, fa, qf, oacc, bias, m_run, l_part,
                                        qpos, a.c, lane);
      attn_walk<DH, true, false, QPRE>(cp, smem, kt_diag, n_kt, n_kt, active, wmax, fa, qf, oacc, bias, m_run,
                                       l_part, qpos, a.c, lane);
    }

    // ---- normalise and store: oacc[db][v] is O[query][db*32 + 8*(v/4) + 4*g + v%4].
    // Feature d = 32*db + 8*vq + 4*g of the head sits in 64-column panel
    // head*DH/64 + db/2 at column 32*(db%2) + 8*vq + 4*g, so every store is a
    // constant offset from one base pointer per lane (a per-column address
    // would be hoisted out of the key walk and spilled).
    const float lsum = halves_sum(l_part);
    const float inv = 1.0f / lsum;
    if constexpr (LSE) {
      // l sums exp2 of the scores (times c unless Q came pre-multiplied) minus
      // the reference max m, which is in the same units as the accumulators
      if (my_valid && g == 0)
        a.lse[(int64_t)head * a.n + qrow] = 0.69314718055994531f * ((QPRE ? m_run : m_run * a.c) + __log2f(lsum));
    }
    if (my_valid) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const float o0 = oacc[db][vq * 4 + 0] * inv, o1 = oacc[db][vq * 4 + 1] * inv;
          const float o2 = oacc[db][vq * 4 + 2] * inv, o3 = oacc[db][vq * 4 + 3] * inv;
          if constexpr (OUT_F32) {
            float *og = reinterpret_cast<float *>(a.o) + qrow * rs + head * DH + g * 4;
            *reinterpret_cast<float4 *>(og + db * 32 + vq * 8) = make_float4(o0, o1, o2, o3);
          } else {
            bf16 *og = reinterpret_cast<bf16 *>(a.o);
            og += a.o_panel ? (int64_t)(head * DH / kPanel + (db >> 1)) * a.o_panel + qrow * kPanel + (db & 1) * 32
                            : qrow * rs + head * DH + db * 32;
            og += g * 4 + vq * 8;
            const bf16x2 w01 = {(bf16)o0, (bf16)o1}, w23 = {(bf16)o2, (bf16)o3};
            u32x2 u = {__builtin_bit_cast(uint32_t, w01), __builtin_bit_cast(uint32_t, w23)};
            *reinterpret_cast<u32x2 *>(og) = u;
          }
        }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
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
  const int64_t rs = (int64_t)a.H * DH, kvs = (int64_t)a.Hkv * DH;  // row pitches: q and o, k and v
  const float *q = reinterpret_cast<const float *>(a.q) + head * DH;
  const float *k = reinterpret_cast<const float *>(a.k) + (head / a.grp) * DH;
  const float *v = reinterpret_cast<const float *>(a.v) + (head / a.grp) * DH;
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
      Ks[tid][d] = key < a.S ? k[key * kvs + d] : 0.f;
      Vs[tid][d] = key < a.S ? v[key * kvs + d] : 0.f;
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
                            bool o_panel, int64_t S, int32_t n, int32_t H, int32_t Hkv, int32_t Dh, float scale,
                            ZigzagMap zz, bool q_prescaled, hipStream_t s, float *lse) {
  if (n <= 0) return hipSuccess;
  if (Hkv < 1 || H % Hkv != 0) return hipErrorInvalidValue;
  if (o_panel && (dtype != TSP_BF16 || o_dtype != TSP_BF16)) return hipErrorInvalidValue;
  if (q_prescaled && (dtype != TSP_BF16 || (o_dtype != TSP_BF16 && !lse))) return hipErrorInvalidValue;
  if (lse && (dtype != TSP_BF16 || o_dtype != TSP_F32)) return hipErrorInvalidValue;
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.S = S;
  a.n = n;
  a.H = H;
  a.Hkv = Hkv;
  a.grp = H / Hkv;
  a.scale = scale;
  // Multiplier of the scores in the exp2 domain. Kept at least the smallest
  // normal float, so that masked scores (-inf) still give 0 with a zero scale;
  // the weights then differ from uniform by under |s| * 2^-126.
  a.c = fmaxf(scale * 1.4426950408889634f, 1.17549435e-38f);
  a.zz = zz;
  a.T = (zz.C + kBQ - 1) / kBQ;
  a.o_panel = o_panel ? (int64_t)n * kPanel : 0;
  a.lse = lse;
  if (dtype == TSP_BF16) {
    dim3 grid(H * a.T);
    const bool f32out = o_dtype == TSP_F32;
    if (lse) {
      if (Dh == 128) {
        if (q_prescaled)
          hipLaunchKernelGGL((attn_bf16_kernel<128, true, true, true>), grid, dim3(kAttnThreads), 0, s, a);
        else
          hipLaunchKernelGGL((attn_bf16_kernel<128, true, false, true>), grid, dim3(kAttnThreads), 0, s, a);
      } else {
        if (q_prescaled)
          hipLaunchKernelGGL((attn_bf16_kernel<64, true, true, true>), grid, dim3(kAttnThreads), 0, s, a);
        else
          hipLaunchKernelGGL((attn_bf16_kernel<64, true, false, true>), grid, dim3(kAttnThreads), 0, s, a);
      }
    } else if (Dh == 128) {
      if (f32out)
        hipLaunchKernelGGL((attn_bf16_kernel<128, true, false>), grid, dim3(kAttnThreads), 0, s, a);
      else if (q_prescaled)
        hipLaunchKernelGGL((attn_bf16_kernel<128, false, true>), grid, dim3(kAttnThreads), 0, s, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<128, false, false>), grid, dim3(kAttnThreads), 0, s, a);
    } else {
      if (f32out)
        hipLaunchKernelGGL((attn_bf16_kernel<64, true, false>), grid, dim3(kAttnThreads), 0, s, a);
      else if (q_prescaled)
        hipLaunchKernelGGL((attn_bf16_kernel<64, false, true>), grid, dim3(kAttnThreads), 0, s, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<64, false, false>), grid, dim3(kAttnThreads), 0, s, a);
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
