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
// Block tile 256 (M) x 256 (N), 4 waves as 2 (M) x 2 (N), one per SIMD, each
// owning 128 x 128 of the output as 4 x 4 MFMA accumulators of 32 x 32. The
// MFMAs produce C^T blocks (B rows are the first operand), so a lane holds 4
// consecutive output columns of one row and every epilogue access is a 16-
// (fp32) or 8-byte (bf16) vector.
// K advances 64 at a time through 2 LDS stages (A and B tiles of 256 x 64,
// 64 KB per stage; the two A tiles, then the two B tiles, so every fragment
// read and copy target is a base register plus an immediate): tiles go from
// HBM straight into LDS (buffer_load ... lds, 16 bytes per lane), one block
// barrier per step, and the loop is unrolled over the two stages. Fragments
// are read two K slices ahead of their MFMAs, so every read of a stage has
// been issued after the second slice of its step; the copies of the step two
// later then go out two per group of MFMAs over the last two slices. Where a
// step's tiles come from is advanced one step at a time in scalar registers
// (the B pointer is read only when a step enters a new segment). Each block
// also pulls its share of the step after that into L2, one dword load per
// 128-byte line: the blocks that run together on one XCD share A and B
// tiles, so each touches only its part of them. LDS rows are 128 bytes; the
// 16-byte chunk index is XOR-swizzled by (row/2)%8 (the copying lane picks
// its source chunk), so the lanes that read one chunk of 32 rows spread over
// all bank groups.
// The A operand may come in the panel layout (64-column panels of [M][64]):
// then one A tile of a step is 32 KB of contiguous memory, which the copy
// engine streams at close to its full rate; from row-major A with a long row
// pitch every copy instruction touches 8 rows far apart and the rate halves.
// fp32 operands use a plain LDS-tiled FMA kernel (64x64 tiles, 4x4 per thread).
#include <algorithm>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "tsp_internal.h"

namespace tsp {

struct GemmArgs {
  const void *A;  // [M][K_total] (lda elements per row), or panel layout
  int64_t lda;
  int64_t a_panel;  // bf16 only: panel stride of A in elements (M_alloc * 64), 0 = row-major
  PtrList B;      // B segments: segment s holds columns [s*kseg, (s+1)*kseg) of B
  int64_t ldb;    // row pitch of every B segment
  int32_t kseg;   // reduction length covered by one B pointer
  int32_t M, N, K;
  int32_t nz;     // independent problems; problem z uses B.p[z] and K == kseg
  // Gated MLP up (epilogue EpiSwiGLU): each B segment holds gate_rows gate
  // rows, then the same units' up rows; the product's N = 2*gate_rows
  // columns interleave them (gemm_bf16_kernel: 64 gate then 64 up columns
  // per 128; the other kernels: gate, up column pairs). 0 otherwise.
  int32_t gate_rows;
};

// B row behind product column v of a gated product (see GemmArgs).
__device__ __forceinline__ int gated_row_blocks(int v, int gate_rows) {
  return ((v >> 7) << 6) + (v & 63) + ((v >> 6) & 1) * gate_rows;
}
__device__ __forceinline__ int gated_row_pairs(int v, int gate_rows) { return (v >> 1) + (v & 1) * gate_rows; }

// ---------------------------------------------------------------- epilogues
// Each epilogue takes one output element (fp32 kernel) or four consecutive
// columns of one row (bf16 kernel) of problem z. On the bf16 kernel's fast
// path it gets a row's whole 128 columns at once (put_row; v[i][vq] holds
// columns 32*i + 8*vq + 4*g .. +3 of the wave's block), which most of them
// store one float4 at a time.
template <class Epi>
__device__ __forceinline__ void put_each(const Epi &e, const typename Epi::Row &w, const float4 (&v)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) e.put(w, i, vq, v[i][vq]);
}
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

// H[:, z*cols + c] = GELU(acc): problem z is ring step z's shard. H is
// row-major with pitch ld, or in panel layout when panel != 0.
template <typename T>
struct EpiGelu {
  T *out;
  int64_t ld;     // row pitch of row-major H
  int64_t panel;  // panel stride of H, or 0
  int32_t cols;   // columns per shard
  __device__ __forceinline__ T *at(int z, int r, int c) const {
    const int64_t col = (int64_t)z * cols + c;
    return out + (panel ? panel_index(r, col, panel) : (int64_t)r * ld + col);
  }
  __device__ __forceinline__ void operator()(int z, int r, int c, float v) const { *at(z, r, c) = (T)gelu_erf(v); }
  __device__ __forceinline__ void operator()(int z, int r, int c, float4 v) const {
    store4(at(z, r, c), make_float4(gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w)));
  }
  // Whole 128-column blocks (see gemm_bf16_kernel): row r, columns c0 + dc
  // with dc = 32*i + 8*vq + 4*g. In panel layout c0 is a multiple of 64, so
  // block half i/2 is panel c0/64 + i/2 and the rest is a constant offset.
  struct Row {
    T *p[2];
  };
  __device__ __forceinline__ bool fast_ok() const { return true; }
  __device__ __forceinline__ Row row(int z, int r, int c0, int g) const {
    const int64_t col = (int64_t)z * cols + c0 + 4 * g;
    Row w;
    if (panel) {
      w.p[0] = out + panel_index(r, col, panel);
      w.p[1] = w.p[0] + panel;
    } else {
      w.p[0] = out + (int64_t)r * ld + col;
      w.p[1] = w.p[0] + 64;
    }
    return w;
  }
  __device__ __forceinline__ void put(const Row &w, int i, int vq, float4 v) const {
    store4(w.p[i >> 1] + (i & 1) * 32 + vq * 8, make_float4(gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w)));
  }
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const { put_each(*this, w, v); }
};

// EpiGelu that also keeps the pre-activation: Z[:, z*cols + c] = acc in bf16,
// row-major with pitch ldz, for a backward that takes Z from the forward.
struct EpiGeluZ {
  EpiGelu<bf16> h;
  bf16 *zo;
  int64_t ldz;
  __device__ __forceinline__ bf16 *zat(int z, int r, int c) const { return zo + (int64_t)r * ldz + (int64_t)z * h.cols + c; }
  __device__ __forceinline__ void operator()(int z, int r, int c, float v) const {
    h(z, r, c, v);
    *zat(z, r, c) = (bf16)v;
  }
  __device__ __forceinline__ void operator()(int z, int r, int c, float4 v) const {
    h(z, r, c, v);
    store4(zat(z, r, c), v);
  }
  struct Row {
    EpiGelu<bf16>::Row hr;
    bf16 *zp;
  };
  __device__ __forceinline__ bool fast_ok() const { return true; }
  __device__ __forceinline__ Row row(int z, int r, int c0, int g) const { return Row{h.row(z, r, c0, g), zat(z, r, c0 + 4 * g)}; }
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        h.put(w.hr, i, vq, v[i][vq]);
        store4(w.zp + i * 32 + vq * 8, v[i][vq]);
      }
  }
};

// H[:, z*cols + u] = SiLU(gate_u) * up_u for hidden unit u of ring step z's
// shard (gated MLP). The fp32 kernel and the leading-rows reduction hand it
// (gate, up) pairs; the bf16 kernel's fast path hands it 128 columns, of
// which blocks i = 0, 1 are the gates and i + 2 the ups of 64 units (B rows
// remapped by gated_row_blocks), all in one lane. 2*cols is a multiple of
// 128, so that path covers every column.
template <typename T>
struct EpiSwiGLU {
  static constexpr bool kGated = true;
  T *out;
  int64_t ld;     // row pitch of row-major H
  int64_t panel;  // panel stride of H, or 0
  int32_t cols;   // hidden units per shard
  __device__ __forceinline__ static float act(float gate, float up) { return silu(gate) * up; }
  __device__ __forceinline__ void pair(int z, int r, int u, float gate, float up) const {
    const int64_t col = (int64_t)z * cols + u;
    out[panel ? panel_index(r, col, panel) : (int64_t)r * ld + col] = (T)act(gate, up);
  }
  struct Row {
    T *p;
  };
  __device__ __forceinline__ bool fast_ok() const { return true; }
  __device__ __forceinline__ Row row(int z, int r, int c0, int g) const {
    const int64_t col = (int64_t)z * cols + (c0 >> 7) * 64;  // first unit of the block, a multiple of 64
    return Row{out + (panel ? panel_index(r, col, panel) : (int64_t)r * ld + col) + 4 * g};
  }
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const float4 a = v[i][vq], b = v[i + 2][vq];
        store4(w.p + i * 32 + vq * 8, make_float4(act(a.x, b.x), act(a.y, b.y), act(a.z, b.z), act(a.w, b.w)));
      }
  }
};

// Whether an epilogue takes gated (gate, up) pairs.
template <class Epi, class = void>
struct is_gated {
  static constexpr bool value = false;
};
template <class Epi>
struct is_gated<Epi, std::void_t<decltype(Epi::kGated)>> {
  static constexpr bool value = Epi::kGated;
};

struct EpiStoreF32 {
  float *out;
  int64_t ld;
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const { out[(int64_t)r * ld + c] = v; }
  __device__ __forceinline__ void operator()(int, int r, int c, float4 v) const {
    *reinterpret_cast<float4 *>(out + (int64_t)r * ld + c) = v;
  }
  struct Row {
    float *p;
  };
  __device__ __forceinline__ bool fast_ok() const { return true; }
  __device__ __forceinline__ Row row(int, int r, int c0, int g) const { return Row{out + (int64_t)r * ld + c0 + 4 * g}; }
  __device__ __forceinline__ void put(const Row &w, int i, int vq, float4 v) const {
    *reinterpret_cast<float4 *>(w.p + i * 32 + vq * 8) = v;
  }
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const { put_each(*this, w, v); }
};

// out [M][N] row-major in bf16, rounded once from the fp32 sums.
struct EpiStoreBf16 {
  bf16 *out;
  int64_t ld;
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const { out[(int64_t)r * ld + c] = (bf16)v; }
  __device__ __forceinline__ void operator()(int, int r, int c, float4 v) const { store4(out + (int64_t)r * ld + c, v); }
  struct Row {
    bf16 *p;
  };
  __device__ __forceinline__ bool fast_ok() const { return true; }
  __device__ __forceinline__ Row row(int, int r, int c0, int g) const { return Row{out + (int64_t)r * ld + c0 + 4 * g}; }
  __device__ __forceinline__ void put(const Row &w, int i, int vq, float4 v) const { store4(w.p + i * 32 + vq * 8, v); }
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const { put_each(*this, w, v); }
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
  struct Row {
    const float *x;
    float *p;
  };
  __device__ __forceinline__ bool fast_ok() const { return true; }
  __device__ __forceinline__ Row row(int, int r, int c0, int g) const {
    const int64_t i = (int64_t)r * ld + c0 + 4 * g;
    return Row{res + i, out + i};
  }
  __device__ __forceinline__ void put(const Row &w, int i, int vq, float4 v) const {
    const int d = i * 32 + vq * 8;
    const float4 x = *reinterpret_cast<const float4 *>(w.x + d);
    *reinterpret_cast<float4 *>(w.p + d) = make_float4(x.x + v.x, x.y + v.y, x.z + v.z, x.w + v.w);
  }
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const { put_each(*this, w, v); }
};

// Shard z of the QKV projection: its output columns are hq Q columns (H/D
// heads), then hk K and hk V columns (Hkv/D heads). Q column c is global
// feature z*hq + c of q [n][ldq], in local row order; K/V column c is feature
// z*hk + c of kf/vf [S][ldkv] at the token's global row. (Four consecutive
// columns never straddle parts: hq and hk are multiples of 4.) ROPE: the
// bf16 fast path rotates Q and K with the table (a separate instance, so that
// the plain one carries no rotation state).
template <typename T, bool ROPE = false>
struct EpiQKV {
  T *q, *k, *v;
  int64_t ldq, ldkv;
  int32_t hq, hk;
  ZigzagMap zz;
  float q_scale;       // factor applied to the Q part before rounding
  const float2 *rope;  // rotary table [local row][dh/2] (cos, sin), or null
  int32_t dh;          // head width (64 or 128) when rope is set
  __device__ __forceinline__ T *dst(int z, int r, int c) const {
    if (c < hq) return q + (int64_t)r * ldq + (int64_t)z * hq + c;
    const int kc = c - hq, part = kc >= hk;
    return (part ? v : k) + (int64_t)zz.pos(r) * ldkv + (int64_t)z * hk + (kc - part * hk);
  }
  __device__ __forceinline__ float factor(int c) const { return c < hq ? q_scale : 1.0f; }
  __device__ __forceinline__ void operator()(int z, int r, int c, float val) const {
    *dst(z, r, c) = (T)(val * factor(c));
  }
  __device__ __forceinline__ void operator()(int z, int r, int c, float4 val) const {
    const float f = factor(c);
    store4(dst(z, r, c), make_float4(val.x * f, val.y * f, val.z * f, val.w * f));
  }
  // whole 128-column blocks stay inside one part when hq and hk are
  // multiples of 128, and then also hold whole heads
  struct Row {
    T *p;
    float f;
    const float2 *rot;  // this row's rotary table when the block is Q or K
  };
  __device__ __forceinline__ bool fast_ok() const { return ((hq | hk) & 127) == 0; }
  __device__ __forceinline__ Row row(int z, int r, int c0, int g) const {
    const bool rotate = ROPE && c0 < hq + hk;
    return Row{dst(z, r, c0 + 4 * g), factor(c0), rotate ? rope + (int64_t)r * (dh / 2) : nullptr};
  }
  __device__ __forceinline__ void put(const Row &w, int i, int vq, float4 v) const {
    store4(w.p + i * 32 + vq * 8, make_float4(v.x * w.f, v.y * w.f, v.z * w.f, v.w * w.f));
  }
  // Rotary embedding on Q and K: feature d of a head pairs with d + dh/2.
  // The block's column 32*i + 8*vq + 4*g + e is feature (32*i) % dh + ...,
  // so block i < its partner i + dh/64 (same vq, same lane) whenever block
  // i holds the first half of a head; the pair's frequency index is
  // (32*i) % (dh/2) + 8*vq + 4*g + e.
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const {
    if (!ROPE || w.rot == nullptr) {
      put_each(*this, w, v);
      return;
    }
    const int step = dh / 64;
    const int g = (threadIdx.x >> 5) & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if ((i / step) & 1) continue;  // second half of a head: handled with its partner
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int f0 = (32 * i) % (dh / 2) + 8 * vq + 4 * g;
        const float4 cs01 = *reinterpret_cast<const float4 *>(w.rot + f0);
        const float4 cs23 = *reinterpret_cast<const float4 *>(w.rot + f0 + 2);
        const float4 a = v[i][vq], b = v[i + step][vq];
        put(w, i, vq,
            make_float4(a.x * cs01.x - b.x * cs01.y, a.y * cs01.z - b.y * cs01.w, a.z * cs23.x - b.z * cs23.y,
                        a.w * cs23.z - b.w * cs23.w));
        put(w, i + step, vq,
            make_float4(b.x * cs01.x + a.x * cs01.y, b.y * cs01.z + a.y * cs01.w, b.z * cs23.x + a.z * cs23.y,
                        b.w * cs23.z + a.w * cs23.w));
      }
    }
  }
};

// ---------------------------------------------------------------- tile order
// ---------------------------------------------------------------- backward epilogues
template <typename T>
__device__ __forceinline__ float4 load4(const T *p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const float4 *>(p);
  } else {
    // a bf16 is the upper half of the fp32 with the same value
    const u32x2 u = *reinterpret_cast<const u32x2 *>(p);
    return make_float4(__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
                       __uint_as_float(u[1] & 0xffff0000u));
  }
}
__device__ __forceinline__ float4 gelu4(float4 v) {
  return make_float4(gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w));
}

// Z^T of the MLP backward: rows are hidden units, columns tokens. zt = Z^T
// (row-major with pitch ld, or panel layout when panel != 0) and ht = GELU(Z^T)
// (row-major, pitch ld), both rounded once from the fp32 product.
template <typename T>
struct EpiZH {
  T *zt, *ht;
  int64_t ld, panel;
  __device__ __forceinline__ T *zat(int r, int c) const {
    return zt + (panel ? panel_index(r, c, panel) : (int64_t)r * ld + c);
  }
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const {
    *zat(r, c) = (T)v;
    ht[(int64_t)r * ld + c] = (T)gelu_erf(v);
  }
  __device__ __forceinline__ void operator()(int, int r, int c, float4 v) const {
    store4(zat(r, c), v);
    store4(ht + (int64_t)r * ld + c, gelu4(v));
  }
  struct Row {
    T *z[2];
    T *h;
  };
  __device__ __forceinline__ bool fast_ok() const { return true; }
  __device__ __forceinline__ Row row(int, int r, int c0, int g) const {
    Row w;
    w.z[0] = zat(r, c0 + 4 * g);
    w.z[1] = panel ? w.z[0] + panel : w.z[0] + 64;
    w.h = ht + (int64_t)r * ld + c0 + 4 * g;
    return w;
  }
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        store4(w.z[i >> 1] + (i & 1) * 32 + vq * 8, v[i][vq]);
        store4(w.h + i * 32 + vq * 8, gelu4(v[i][vq]));
      }
  }
};

// dZ^T = acc * GELU'(Z^T), in place over the Z^T buffer of EpiZH (each
// element is read and then written by the same lane).
template <typename T>
struct EpiDZ {
  T *zt;
  int64_t ld, panel;
  __device__ __forceinline__ T *zat(int r, int c) const {
    return zt + (panel ? panel_index(r, c, panel) : (int64_t)r * ld + c);
  }
  __device__ __forceinline__ static float4 dz4(float4 v, float4 z) {
    return make_float4(v.x * gelu_erf_grad(z.x), v.y * gelu_erf_grad(z.y), v.z * gelu_erf_grad(z.z),
                       v.w * gelu_erf_grad(z.w));
  }
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const {
    T *p = zat(r, c);
    *p = (T)(v * gelu_erf_grad((float)*p));
  }
  __device__ __forceinline__ void operator()(int, int r, int c, float4 v) const {
    T *p = zat(r, c);
    store4(p, dz4(v, load4(p)));
  }
  struct Row {
    T *z[2];
  };
  __device__ __forceinline__ bool fast_ok() const { return true; }
  __device__ __forceinline__ Row row(int, int r, int c0, int g) const {
    Row w;
    w.z[0] = zat(r, c0 + 4 * g);
    w.z[1] = panel ? w.z[0] + panel : w.z[0] + 64;
    return w;
  }
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        T *p = w.z[i >> 1] + (i & 1) * 32 + vq * 8;
        store4(p, dz4(v[i][vq], load4(p)));
      }
  }
};

// fp32 weight gradient split over shards: by rows (row m -> shard m / split,
// pitch ld) or by columns (column c -> shard c / split, pitch split).
struct EpiShardF32 {
  PtrList out;
  int32_t split;
  int64_t ld;
  bool by_rows;
  __device__ __forceinline__ float *at(int r, int c) const {
    if (by_rows) return (float *)out.p[r / split] + (int64_t)(r % split) * ld + c;
    return (float *)out.p[c / split] + (int64_t)r * split + (c % split);
  }
  __device__ __forceinline__ void operator()(int, int r, int c, float v) const { *at(r, c) = v; }
  __device__ __forceinline__ void operator()(int, int r, int c, float4 v) const {
    *reinterpret_cast<float4 *>(at(r, c)) = v;  // split % 4 == 0: never straddles shards
  }
  struct Row {
    float *p;
  };
  // a wave's 128 columns (c0 a multiple of 128) stay in one shard
  __device__ __forceinline__ bool fast_ok() const { return by_rows || (split & 127) == 0; }
  __device__ __forceinline__ Row row(int, int r, int c0, int g) const { return Row{at(r, c0 + 4 * g)}; }
  __device__ __forceinline__ void put(const Row &w, int i, int vq, float4 v) const {
    *reinterpret_cast<float4 *>(w.p + i * 32 + vq * 8) = v;
  }
  __device__ __forceinline__ void put_row(const Row &w, const float4 (&v)[4][4]) const { put_each(*this, w, v); }
};

// Logical tile L -> (z, tm, tn): problems outermost, then groups of GM tile
// rows walked column-major, so the blocks that run together on one XCD share
// A row panels and B column panels in its L2.
struct TileCoord {
  int z, tm, tn;
};
constexpr int kTileGM = 4;    // tile rows per group
constexpr int kXcdBlocks = 32;  // blocks that run together on one XCD (its CUs, one block each)
__device__ __forceinline__ TileCoord tile_of(int L, int tiles_m, int tiles_n) {
  constexpr int GM = kTileGM;
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
constexpr int kBM = 256, kBN = 256, kBK = 64, kGemmThreads = 256, kGemmStages = 2;
constexpr int kRowBytes = kBK * 2;                              // 128: one cache line per tile row and step
constexpr int kTileBytes = kBM * kRowBytes;                     // one 256 x 64 bf16 tile: 32 KB
constexpr int kGemmStageBytes = 2 * kTileBytes;                 // A tile + B tile
constexpr size_t kGemmLds = (size_t)kGemmStages * kGemmStageBytes;  // 128 KB
constexpr int kGemmWaves = kGemmThreads / 64;
// 1 KB copy windows per wave, per tile; 16-wide K slices per step
[[maybe_unused]] constexpr int kWinPerWave = kTileBytes / 1024 / kGemmWaves;
[[maybe_unused]] constexpr int kGemmSlices = kBK / 16;

// Byte offset of logical 16-byte chunk ch (0..7) of row r in a 128-byte-row
// tile: the 16 rows that 16 lanes read with one logical chunk land in 16
// distinct bank groups.
__device__ __forceinline__ int gswz(int r, int ch) { return r * kRowBytes + ((ch ^ ((r >> 1) & 7)) << 4); }

// Fragments of one 16-wide K slice for a wave's 128 x 128 output: 4 A row
// blocks (M) and 4 B row blocks (N) of 32.
struct GemmFrags {
  bf16x8 a[4], b[4];
};

// One 16-byte-per-lane copy into LDS at sbase + IMM (lane i -> +16*i); M0 is
// set with one add. Same contract as lds_copy16.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int IMM>
__device__ __forceinline__ void lds_copy16_at(u32x4 rsrc, int voffset, int soffset, uint32_t sbase) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile(
      "s_add_u32 m0, %3, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "s"(soffset), "s"(sbase), "n"(IMM)
      : "memory", "m0", "scc");
#endif
}
#pragma clang diagnostic pop

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <class Epi>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(GemmArgs a, Epi epi) {
#if defined(__HIP_DEVICE_COMPILE__)
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr bool kGatedB = is_gated<Epi>::value;

  const int tiles_m = (a.M + kBM - 1) / kBM, tiles_n = (a.N + kBN - 1) / kBN;
  const TileCoord tc = tile_of(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n);
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN, z = tc.z;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // wave tile: rows wm*128.., columns wn*128..
  const int g = lane >> 5, l32 = lane & 31;

  // LDS: the A tiles of stages 0 and 1, then the B tiles of stages 0 and 1
  // (32 KB each), so every fragment read and copy target of a stage is a
  // base plus an immediate below 64 KB.
  // ---- copy plan: each wave copies windows kWinPerWave*wave.. of the A and
  // B tiles of a step; window w = tile rows 8w..8w+7 (1 KB). Lane -> (row,
  // chunk position); it loads the logical chunk that belongs there.
  const uint32_t wbase = lds_addr(smem) + kWinPerWave * wave * 1024;
  const bool a_panel = a.a_panel != 0;
  const int64_t a_pitch = a_panel ? kPanel : a.lda;  // elements between A rows
  int a_off[kWinPerWave], b_off[kWinPerWave];
#pragma unroll
  for (int i = 0; i < kWinPerWave; ++i) {
    const int win = kWinPerWave * wave + i, row = win * 8 + lane / 8, pos = lane & 7;
    const int ch = pos ^ ((row >> 1) & 7);
    a_off[i] = (int)(row * a_pitch * 2) + ch * 16;
    if constexpr (kGatedB)  // offset from the segment start (descriptor below)
      b_off[i] = (int)(gated_row_blocks(n0 + row, a.gate_rows) * a.ldb * 2) + ch * 16;
    else
      b_off[i] = (int)(row * a.ldb * 2) + ch * 16;
  }
  const int a_rows = min(kBM, a.M - m0), b_rows = min(kBN, a.N - n0);
  const bf16 *Ab = reinterpret_cast<const bf16 *>(a.A) + (int64_t)m0 * a_pitch;

  // B segment pointers are read from LDS when a step enters a new segment: a
  // scalar load would turn every wait on the LDS counter into a full wait.
  __shared__ uint64_t bptr_s[TSP_MAX_D];
  if (tid < TSP_MAX_D) bptr_s[tid] = (uint64_t)(uintptr_t)a.B.p[tid];
  auto bptr_at = [&](int seg) {
    const uint64_t v = bptr_s[seg];
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    return reinterpret_cast<const bf16 *>((uintptr_t)(((uint64_t)hi << 32) | lo));
  };
  auto b_rsrc = [&](const bf16 *bseg) {
    if constexpr (kGatedB)  // the tile's rows are spread over the gate and up halves
      return buffer_rsrc(bseg, (uint32_t)(2 * a.gate_rows * a.ldb * 2));
    else
      return buffer_rsrc(bseg + (int64_t)n0 * a.ldb, (uint32_t)(b_rows * a.ldb * 2));
  };
  // Where a step's tiles come from, advanced one step at a time: row-major A
  // keeps one descriptor over the block's rows and moves along K with
  // soffset; panel A moves the descriptor base by one panel; B moves along K
  // with soffset inside a segment and takes the next segment's descriptor at
  // its start.
  struct StepSrc {
    u32x4 ar, br;
    int a_soff, b_soff;
    const bf16 *a_base;
    int kt, seg, koff;
  };
  auto src_at = [&](int kt) {
    StepSrc t;
    t.kt = kt;
    const int k0 = kt * kBK;
    t.seg = a.nz > 1 ? z : k0 / a.kseg;
    t.koff = a.nz > 1 ? k0 : k0 - t.seg * a.kseg;
    t.br = b_rsrc(reinterpret_cast<const bf16 *>(a.B.p[t.seg]));
    t.b_soff = t.koff * 2;
    if (a_panel) {
      t.a_base = Ab + (int64_t)kt * a.a_panel;
      t.ar = buffer_rsrc(t.a_base, (uint32_t)(a_rows * kRowBytes));
      t.a_soff = 0;
    } else {
      t.a_base = Ab;
      t.ar = buffer_rsrc(Ab, (uint32_t)(a_rows * a_pitch * 2));
      t.a_soff = k0 * 2;
    }
    return t;
  };
  // next step, or the same one past the last step (its copies then land in
  // a stage nobody reads again)
  const int KT = a.K / kBK;
  auto advance = [&](StepSrc &t) {
    if (t.kt + 1 >= KT) return;
    ++t.kt;
    if (a_panel) {
      t.a_base += a.a_panel;
      t.ar = buffer_rsrc(t.a_base, (uint32_t)(a_rows * kRowBytes));
    } else {
      t.a_soff += kBK * 2;
    }
    t.koff += kBK;
    if (a.nz == 1 && t.koff >= a.kseg) {
      t.koff -= a.kseg;
      ++t.seg;
      t.br = b_rsrc(bptr_at(t.seg));
    }
    t.b_soff = t.koff * 2;
  };
  // copies of window Q of the A and B tiles of source t into stage ST
  auto copy_win = [&](const StepSrc &t, auto stc, auto qc) {
    constexpr int ST = decltype(stc)::value, Q = decltype(qc)::value;
    lds_copy16_at<ST * kTileBytes + Q * 1024>(t.ar, a_off[Q], t.a_soff, wbase);
    lds_copy16_at<(2 + ST) * kTileBytes + Q * 1024>(t.br, b_off[Q], t.b_soff, wbase);
  };
  // L2 prefetch of a step's tiles, one dword load per 128-byte line into a
  // scratch LDS area that nobody reads. The blocks that run together on one
  // XCD come in groups of kTileGM tile rows walked column-major (tile_of):
  // about min(tiles_n, kXcdBlocks / kTileGM) of them share each A tile and
  // the group's rows share each B tile, so a block touches only its share of
  // each, A rows with waves 0 and 2 and B rows with waves 1 and 3 (up to 128
  // rows each). Lanes outside the share get an offset past the buffer and
  // touch nothing; every wave still issues both loads, so the wait counts
  // stay uniform.
  __shared__ uint32_t pf_sink[64];
  const uint32_t sink = lds_addr(pf_sink);
  constexpr int kOut = 0x7fffff00;  // past any buffer range
  const int share_a = min(tiles_n, kXcdBlocks / kTileGM), rows_a = (kBM + share_a - 1) / share_a;
  const int first_m = tc.tm - tc.tm % kTileGM, share_b = min(tiles_m - first_m, kTileGM);
  const int rows_b = (kBN + share_b - 1) / share_b;
  const int pf_r = lane + ((wave >> 1) << 6);  // waves 0, 1: 0..63; waves 2, 3: 64..127
  const int pf_arow = (tc.tn % share_a) * rows_a + pf_r, pf_brow = (tc.tm - first_m) * rows_b + pf_r;
  const bool pf_aok = (wave & 1) == 0 && pf_r < rows_a && pf_arow < kBM;
  const bool pf_bok = (wave & 1) == 1 && pf_r < rows_b && pf_brow < kBN;
  const int pf_va = pf_aok ? pf_arow * (int)(a_pitch * 2) : kOut;
  const int pf_vb =
      pf_bok ? (kGatedB ? gated_row_blocks(n0 + pf_brow, a.gate_rows) : pf_brow) * (int)(a.ldb * 2) : kOut;
  auto prefetch = [&](const StepSrc &t) {
    lds_touch4(t.ar, pf_va, t.a_soff, sink);
    lds_touch4(t.br, pf_vb, t.b_soff, sink);
  };

  // fragment read bases for K slice kk: A rows wm*128 + l32, B rows wn*128 +
  // l32, chunk 2*kk + g; block i of 32 rows and the stage are immediates (the
  // swizzle depends on the row modulo 16 only)
  const unsigned char *fa_a[kGemmSlices], *fa_b[kGemmSlices];
#pragma unroll
  for (int kk = 0; kk < kGemmSlices; ++kk) {
    fa_a[kk] = smem + gswz(wm * 128 + l32, 2 * kk + g);
    fa_b[kk] = smem + 2 * kTileBytes + gswz(wn * 128 + l32, 2 * kk + g);
  }
  // fragment pair q of K slice kk: q = 0, 1 -> A blocks 2q, 2q+1; q = 2, 3 ->
  // B blocks 2q-4, 2q-3 (the first MFMA row of a slice needs every A block)
  auto read_pair = [&](GemmFrags &f, auto stc, int kk, int q) {
    constexpr int ST = decltype(stc)::value;
    if (q < 2) {
      f.a[2 * q] = *reinterpret_cast<const bf16x8 *>(fa_a[kk] + ST * kTileBytes + (2 * q) * 32 * kRowBytes);
      f.a[2 * q + 1] = *reinterpret_cast<const bf16x8 *>(fa_a[kk] + ST * kTileBytes + (2 * q + 1) * 32 * kRowBytes);
    } else {
      f.b[2 * q - 4] = *reinterpret_cast<const bf16x8 *>(fa_b[kk] + ST * kTileBytes + (2 * q - 4) * 32 * kRowBytes);
      f.b[2 * q - 3] = *reinterpret_cast<const bf16x8 *>(fa_b[kk] + ST * kTileBytes + (2 * q - 3) * 32 * kRowBytes);
    }
  };

  f32x16 acc[4][4];  // acc[i][j]: C^T block (N block i, M block j)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto mfma_row = [&](const GemmFrags &f, int i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[i], f.a[j], acc[i][j], 0, 0, 0);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // ---- prologue: steps 0 and 1 into stages 0 and 1, step 2 towards L2.
  StepSrc cs = src_at(0);
  static_for<kWinPerWave>([&](auto q) { copy_win(cs, S0{}, q); });
  __syncthreads();  // bptr_s visible before advance() may read it
  advance(cs);
  static_for<kWinPerWave>([&](auto q) { copy_win(cs, S1{}, q); });
  advance(cs);  // step 2: copied under step 0, which then moves on to step 3 and prefetches it
  prefetch(cs);
  wait_vmcnt<2>();
  __syncthreads();
  // fragments two K slices ahead: slice s of a step uses f[s]
  GemmFrags f[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) read_pair(f[0], S0{}, 0, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) read_pair(f[1], S0{}, 1, q);

  // ---- one step in stage ST. Slice s runs as 4 groups of 4 MFMAs on f[s];
  // slices 0 and 1 read slices 2 and 3 of this step, slices 2 and 3 read
  // slices 0 and 1 of the next. After slice 1 every read of stage ST has
  // been issued: the wave waits for them and for its copies of the next step,
  // and the block synchronises; the copies of the step two later into stage
  // ST then go out two per MFMA group over slices 2 and 3; the source then
  // moves on one step, which is prefetched into L2.
  auto step = [&](auto stc) {
    constexpr int ST = decltype(stc)::value;
    using SN = std::integral_constant<int, 1 - ST>;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      read_pair(f[2], stc, 2, i);
      mfma_row(f[0], i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      read_pair(f[3], stc, 3, i);
      mfma_row(f[1], i);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<2>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    static_for<4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      read_pair(f[0], SN{}, 0, i);
      copy_win(cs, stc, std::integral_constant<int, i>{});
      mfma_row(f[2], i);
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      read_pair(f[1], SN{}, 1, i);
      copy_win(cs, stc, std::integral_constant<int, 4 + i>{});
      if constexpr (i == 3) {
        advance(cs);
        prefetch(cs);
      }
      mfma_row(f[3], i);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    step(S0{});
    step(S1{});
  }
  if (kt < KT) step(S0{});
  // no copy may still be landing in LDS when the block exits
  wait_vmcnt<0>();

  // accumulator layout (C^T block): lane holds output row (M) l32 of the
  // block and columns (N) 8*(v/4) + 4*g + v%4
  // When the wave's 128 columns all lie inside N, each row's addresses come
  // from one per-row base plus constant offsets.
  const int c0 = n0 + wn * 128;
  const bool whole = c0 + 128 <= a.N && epi.fast_ok();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = m0 + wm * 128 + j * 32 + l32;
    if (row >= a.M) continue;
    if (whole) {
      const typename Epi::Row rw = epi.row(z, row, c0, g);
      float4 vals[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq)
          vals[i][vq] = make_float4(acc[i][j][vq * 4 + 0], acc[i][j][vq * 4 + 1], acc[i][j][vq * 4 + 2],
                                    acc[i][j][vq * 4 + 3]);
      epi.put_row(rw, vals);
    } else if constexpr (!kGatedB) {  // gated: every wave's 128 columns are whole or past N
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const int col = c0 + i * 32 + vq * 8 + g * 4;
          if (col < a.N)
            epi(z, row, col,
                make_float4(acc[i][j][vq * 4 + 0], acc[i][j][vq * 4 + 1], acc[i][j][vq * 4 + 2],
                            acc[i][j][vq * 4 + 3]));
        }
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
    if (n0 + lrow < a.N) {
      const int brow = is_gated<Epi>::value ? gated_row_pairs(n0 + lrow, a.gate_rows) : n0 + lrow;
      bv = *reinterpret_cast<const float4 *>(B + (int64_t)brow * a.ldb + koff + lk);
    }
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
  if constexpr (is_gated<Epi>::value) {
    // columns 2u, 2u+1 are the gate and up of unit u (N is even)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const int r = m0 + ty * 4 + i, c = n0 + tx * 4 + j;
        if (r < a.M && c < a.N) epi.pair(z, r, c >> 1, acc[i][j], acc[i][j + 1]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = m0 + ty * 4 + i, c = n0 + tx * 4 + j;
        if (r < a.M && c < a.N) epi(z, r, c, acc[i][j]);
      }
  }
}

// ---------------------------------------------------------------- leading rows
// C = A B^T for at most kLeadRows rows with fp32 A and bf16 B, accurate to
// fp32 level: A is split into bf16 hi + lo (A - hi is exact in fp32, and lo
// keeps it to 2^-9 of itself, so A = hi + lo to about 2^-17 relative), and B
// is exactly bf16, so hi B^T + lo B^T on the matrix cores, accumulated in
// fp32, reproduces the fp32 product. The few rows make this a weight stream:
// each wave owns 32 columns and one K chunk for all rows (two 32-row MFMA
// blocks), so every weight is read once, and the block's 4 waves share each
// 64-wide slab of A (split once) through LDS. The K chunks' partial sums go
// to part[chunk][row][z*N + column] and a second kernel adds them in chunk
// order (deterministic) and applies the epilogue.
// Largest chunk of 512, 256, 128 or 64 that divides the segment length.
static int lead_chunk(int kseg) {
  for (int c = 512; c > 64; c >>= 1)
    if (kseg % c == 0) return c;
  return 64;
}

__global__ __launch_bounds__(256) void lead_gemm_kernel(GemmArgs a, int chunk, float *__restrict__ part) {
#if defined(__HIP_DEVICE_COMPILE__)
  // one 64-wide K slab of A for all 64 rows, split into bf16 hi and lo and
  // shared by the block's 4 waves; rows padded by 16 bytes so that the
  // fragment reads of 32 consecutive rows spread over the banks
  constexpr int kSlab = 64, kPitch = kSlab + 8;
  __shared__ __attribute__((aligned(16))) bf16 Ah[kLeadRows * kPitch], Al[kLeadRows * kPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int groups = (a.N + 127) / 128;  // 4 waves x 32 columns per block
  const int z = blockIdx.x / groups;
  const int n0 = (blockIdx.x - z * groups) * 128 + wave * 32;
  const int kc = blockIdx.y, k_begin = kc * chunk;
  int seg, koff;
  if (a.nz > 1) {
    seg = z;
    koff = k_begin;
  } else {
    seg = k_begin / a.kseg;
    koff = k_begin - seg * a.kseg;
  }
  const int l32 = lane & 31, g = lane >> 5;
  // lane: B row n (column of C), A rows l32 and 32 + l32, K elements 8g..8g+7
  // of each 16-wide slice. Lanes past N read row 0 instead: their products
  // land only in columns of C that are not stored (likewise A rows past M).
  const int n = n0 + l32;
  const bool n_ok = n < a.N;
  const int nrow = !n_ok ? 0 : a.gate_rows ? gated_row_pairs(n, a.gate_rows) : n;
  const bf16 *brow = reinterpret_cast<const bf16 *>(a.B.p[seg]) + (int64_t)nrow * a.ldb + koff + 8 * g;
  // slab staging: thread -> A row tid/4, 16 consecutive K elements
  const int sr = tid >> 2, sk = (tid & 3) * 16;
  const float *asrc = reinterpret_cast<const float *>(a.A) + (int64_t)(sr < a.M ? sr : 0) * a.lda + k_begin + sk;
  f32x16 acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc0[v] = acc1[v] = 0.f;
  for (int k = 0; k < chunk; k += kSlab) {
    bf16x8 wf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) wf[t] = *reinterpret_cast<const bf16x8 *>(brow + k + 16 * t);
    float4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const float4 *>(asrc + k + 4 * i);
    __syncthreads();  // the previous slab's fragments are read
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const float v[8] = {x[i].x, x[i].y, x[i].z, x[i].w, x[i + 1].x, x[i + 1].y, x[i + 1].z, x[i + 1].w};
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 h2 = {(bf16)v[e], (bf16)v[e + 1]};
        const bf16x2 l2 = {(bf16)(v[e] - (float)h2[0]), (bf16)(v[e + 1] - (float)h2[1])};
        hi[e] = h2[0];
        hi[e + 1] = h2[1];
        lo[e] = l2[0];
        lo[e + 1] = l2[1];
      }
      *reinterpret_cast<bf16x8 *>(&Ah[sr * kPitch + sk + 4 * i]) = hi;
      *reinterpret_cast<bf16x8 *>(&Al[sr * kPitch + sk + 4 * i]) = lo;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = 16 * t + 8 * g;
      const bf16x8 h0 = *reinterpret_cast<const bf16x8 *>(&Ah[l32 * kPitch + c]);
      const bf16x8 o0 = *reinterpret_cast<const bf16x8 *>(&Al[l32 * kPitch + c]);
      const bf16x8 h1 = *reinterpret_cast<const bf16x8 *>(&Ah[(32 + l32) * kPitch + c]);
      const bf16x8 o1 = *reinterpret_cast<const bf16x8 *>(&Al[(32 + l32) * kPitch + c]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h0, wf[t], acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o0, wf[t], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h1, wf[t], acc1, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o1, wf[t], acc1, 0, 0, 0);
    }
  }
  // acc[v] is C[8*(v/4) + 4g + v%4 (+32 for acc1)][n]
  if (!n_ok) return;
  const int64_t ntot = (int64_t)a.nz * a.N;
  float *pc = part + (int64_t)kc * a.M * ntot + (int64_t)z * a.N + n;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v >> 2) + 4 * g + (v & 3);
    if (r < a.M) pc[r * ntot] = acc0[v];
    if (r + 32 < a.M) pc[(r + 32) * ntot] = acc1[v];
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <class Epi>
__global__ __launch_bounds__(256) void lead_reduce_kernel(int32_t M, int32_t N, int32_t nz, int32_t chunks,
                                                          const float *__restrict__ part, Epi epi) {
  const int64_t ntot = (int64_t)nz * N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if constexpr (is_gated<Epi>::value) {  // one thread per (row, unit): columns 2u, 2u+1
    if (i >= M * (ntot >> 1)) return;
    const int r = (int)(i / (ntot >> 1));
    const int64_t zc = 2 * (i - r * (ntot >> 1));
    const int z = (int)(zc / N), c = (int)(zc - (int64_t)z * N);
    float gate = 0.f, up = 0.f;
    for (int kc = 0; kc < chunks; ++kc) {
      gate += part[((int64_t)kc * M + r) * ntot + zc];
      up += part[((int64_t)kc * M + r) * ntot + zc + 1];
    }
    epi.pair(z, r, c >> 1, gate, up);
  } else {
    if (i >= M * ntot) return;
    const int r = (int)(i / ntot);
    const int64_t zc = i - r * ntot;
    const int z = (int)(zc / N), c = (int)(zc - (int64_t)z * N);
    float v = 0.f;
    for (int kc = 0; kc < chunks; ++kc) v += part[((int64_t)kc * M + r) * ntot + zc];
    epi(z, r, c, v);
  }
}

template <class Epi>
static hipError_t run_lead(const GemmArgs &a, const Epi &epi, float *part, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.M > kLeadRows) return hipErrorInvalidValue;
  const int chunk = lead_chunk(a.kseg);
  const int chunks = a.K / chunk;
  dim3 grid(a.nz * ((a.N + 127) / 128), chunks);
  hipLaunchKernelGGL(lead_gemm_kernel, grid, dim3(256), 0, s, a, chunk, part);
  const int64_t total = (int64_t)a.M * a.nz * a.N;
  hipLaunchKernelGGL((lead_reduce_kernel<Epi>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a.M, a.N,
                     a.nz, chunks, (const float *)part, epi);
  return hipGetLastError();
}

static GemmArgs lead_args(const float *A, int64_t lda, int32_t M, int32_t N, int32_t K) {
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

size_t lead_part_bytes(int32_t m, int32_t h, int32_t F, int32_t D, bool gated) {
  const int32_t hd = h / D, fd = F / D;
  const size_t qkv = (size_t)(h / lead_chunk(h)) * m * 3 * h;
  const size_t op = (size_t)(h / lead_chunk(hd)) * m * h;
  const size_t up = (size_t)(h / lead_chunk(h)) * m * (gated ? 2 * F : F);
  const size_t dn = (size_t)(F / lead_chunk(fd)) * m * h;
  return 4 * std::max(std::max(qkv, op), std::max(up, dn));
}

hipError_t launch_lead_qkv(const float *a, int32_t m, int32_t h, const PtrList &w, int32_t D, int32_t hq, int32_t hk,
                           float *q, float *k, float *v, ZigzagMap zz, float *part, hipStream_t s) {
  GemmArgs g = lead_args(a, h, m, hq + 2 * hk, h);
  g.B = w;
  g.ldb = h;
  g.nz = D;
  EpiQKV<float> e{q, k, v, (int64_t)D * hq, (int64_t)D * hk, hq, hk, zz, 1.0f, nullptr, 0};
  return run_lead(g, e, part, s);
}

hipError_t launch_lead_outproj(const float *o, int32_t m, int32_t h, const PtrList &wo, int32_t D, int32_t hd,
                               const float *x, float *y, float *part, hipStream_t s) {
  GemmArgs g = lead_args(o, h, m, h, D * hd);
  g.B = wo;
  g.ldb = hd;
  g.kseg = hd;
  EpiAddF32 e{x, y, h};
  return run_lead(g, e, part, s);
}

hipError_t launch_lead_mlp_up(const float *a, int32_t m, int32_t h, const PtrList &w1, int32_t D, int32_t fd,
                              bool gated, float *hid, float *part, hipStream_t s) {
  GemmArgs g = lead_args(a, h, m, gated ? 2 * fd : fd, h);
  g.B = w1;
  g.ldb = h;
  g.nz = D;
  if (gated) {
    g.gate_rows = fd;
    EpiSwiGLU<float> e{hid, (int64_t)D * fd, 0, fd};
    return run_lead(g, e, part, s);
  }
  EpiGelu<float> e{hid, (int64_t)D * fd, 0, fd};
  return run_lead(g, e, part, s);
}

hipError_t launch_lead_mlp_down(const float *hid, int32_t m, const PtrList &w2, int32_t D, int32_t fd, int32_t h,
                                const float *res, float *y, float *part, hipStream_t s) {
  GemmArgs g = lead_args(hid, (int64_t)D * fd, m, h, D * fd);
  g.B = w2;
  g.ldb = fd;
  g.kseg = fd;
  EpiAddF32 e{res, y, h};
  return run_lead(g, e, part, s);
}

// ---------------------------------------------------------------- launchers
template <class Epi>
static hipError_t run_gemm(int dtype, const GemmArgs &a, const Epi &epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.a_panel && dtype != TSP_BF16) return hipErrorInvalidValue;
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

// a_panel: A in panel layout with M rows (bf16 only).
static GemmArgs make_args(const void *A, int64_t lda, bool a_panel, int32_t M, int32_t N, int32_t K) {
  GemmArgs a{};
  a.A = A;
  a.lda = lda;
  a.a_panel = a_panel ? (int64_t)M * kPanel : 0;
  a.M = M;
  a.N = N;
  a.K = K;
  a.kseg = K;
  a.nz = 1;
  return a;
}

hipError_t launch_qkv(int dtype, const void *xn, bool a_panel, int32_t n, int32_t h, const PtrList &w, int32_t D,
                      int32_t hq, int32_t hk, void *q, void *kf, void *vf, ZigzagMap zz, float q_scale,
                      const float2 *rope, int32_t Dh, hipStream_t s) {
  if (rope != nullptr && (dtype != TSP_BF16 || ((hq | hk) & 127) != 0)) return hipErrorInvalidValue;
  GemmArgs a = make_args(xn, h, a_panel, n, hq + 2 * hk, h);
  a.B = w;
  a.ldb = h;
  a.nz = D;
  const int64_t ldq = (int64_t)D * hq, ldkv = (int64_t)D * hk;
  if (dtype == TSP_BF16) {
    if (rope != nullptr) {
      EpiQKV<bf16, true> e{(bf16 *)q, (bf16 *)kf, (bf16 *)vf, ldq, ldkv, hq, hk, zz, q_scale, rope, Dh};
      return run_gemm(dtype, a, e, s);
    }
    EpiQKV<bf16> e{(bf16 *)q, (bf16 *)kf, (bf16 *)vf, ldq, ldkv, hq, hk, zz, q_scale, nullptr, 0};
    return run_gemm(dtype, a, e, s);
  }
  EpiQKV<float> e{(float *)q, (float *)kf, (float *)vf, ldq, ldkv, hq, hk, zz, q_scale, nullptr, 0};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_outproj(int dtype, const void *o, bool a_panel, int32_t n, int32_t h, const PtrList &wo,
                          int32_t D, int32_t hd, const float *x, float *y, hipStream_t s) {
  GemmArgs a = make_args(o, h, a_panel, n, h, D * hd);
  a.B = wo;
  a.ldb = hd;
  a.kseg = hd;
  EpiAddF32 e{x, y, h};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_mlp_up(int dtype, const void *x, bool a_panel, int32_t n, int32_t h, const PtrList &w1, int32_t D,
                         int32_t fd, bool gated, void *hid, bool hid_panel, hipStream_t s, void *z_out) {
  GemmArgs a = make_args(x, h, a_panel, n, gated ? 2 * fd : fd, h);
  a.B = w1;
  a.ldb = h;
  a.nz = D;
  const int64_t hp = hid_panel ? (int64_t)n * kPanel : 0;
  if (gated) {
    // the gated bf16 path needs whole 128-column blocks and 32-bit B offsets
    if ((fd & 63) != 0 || (int64_t)(2 * fd + 256) * h * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    a.gate_rows = fd;
    if (dtype == TSP_BF16) {
      EpiSwiGLU<bf16> e{(bf16 *)hid, (int64_t)D * fd, hp, fd};
      return run_gemm(dtype, a, e, s);
    }
    EpiSwiGLU<float> e{(float *)hid, (int64_t)D * fd, hp, fd};
    return run_gemm(dtype, a, e, s);
  }
  if (z_out != nullptr) {
    if (dtype != TSP_BF16) return hipErrorInvalidValue;
    EpiGeluZ e{EpiGelu<bf16>{(bf16 *)hid, (int64_t)D * fd, hp, fd}, (bf16 *)z_out, (int64_t)D * fd};
    return run_gemm(dtype, a, e, s);
  }
  if (dtype == TSP_BF16) {
    EpiGelu<bf16> e{(bf16 *)hid, (int64_t)D * fd, hp, fd};
    return run_gemm(dtype, a, e, s);
  }
  EpiGelu<float> e{(float *)hid, (int64_t)D * fd, hp, fd};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_mlp_down(int dtype, const void *hid, bool a_panel, int32_t n, const PtrList &w2, int32_t D,
                           int32_t fd, int32_t h, const float *res, float *y, hipStream_t s) {
  GemmArgs a = make_args(hid, (int64_t)D * fd, a_panel, n, h, D * fd);
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

// ---------------------------------------------------------------- MLP backward
hipError_t launch_mlp_bwd_recompute(int dtype, const void *w1cat, int32_t F, int32_t h, const void *x, int32_t n,
                                    void *zt, bool zt_panel, void *ht, hipStream_t s) {
  GemmArgs a = make_args(w1cat, h, false, F, n, h);
  a.B.p[0] = x;
  a.ldb = h;
  const int64_t pnl = zt_panel ? (int64_t)F * kPanel : 0;
  if (dtype == TSP_BF16) {
    EpiZH<bf16> e{(bf16 *)zt, (bf16 *)ht, n, pnl};
    return run_gemm(dtype, a, e, s);
  }
  EpiZH<float> e{(float *)zt, (float *)ht, n, pnl};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_mlp_bwd_dz(int dtype, const void *w2t, int32_t F, int32_t h, const void *dy, int32_t n, void *zt,
                             bool zt_panel, hipStream_t s) {
  GemmArgs a = make_args(w2t, h, false, F, n, h);
  a.B.p[0] = dy;
  a.ldb = h;
  const int64_t pnl = zt_panel ? (int64_t)F * kPanel : 0;
  if (dtype == TSP_BF16) {
    EpiDZ<bf16> e{(bf16 *)zt, n, pnl};
    return run_gemm(dtype, a, e, s);
  }
  EpiDZ<float> e{(float *)zt, n, pnl};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_wgrad(int dtype, const void *A, bool a_panel, int32_t M, const void *b, int32_t N, int32_t n,
                        const PtrList &out, int32_t split, bool by_rows, hipStream_t s) {
  if (split <= 0 || (split & 3) != 0) return hipErrorInvalidValue;
  GemmArgs a = make_args(A, n, a_panel, M, N, n);
  a.B.p[0] = b;
  a.ldb = n;
  EpiShardF32 e{out, split, N, by_rows};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_mlp_bwd_dx(int dtype, const void *dz, bool a_panel, int32_t n, int32_t F, const void *w1t,
                             int32_t h, const float *res, float *dx, hipStream_t s) {
  GemmArgs a = make_args(dz, F, a_panel, n, h, F);
  a.B.p[0] = w1t;
  a.ldb = F;
  if (res) {
    EpiAddF32 e{res, dx, h};
    return run_gemm(dtype, a, e, s);
  }
  EpiStoreF32 e{dx, h};
  return run_gemm(dtype, a, e, s);
}

hipError_t launch_gemm_nt(int dtype, const void *A, bool a_panel, int32_t M, int32_t K, const void *B, int32_t N,
                          void *out, int out_dtype, hipStream_t s) {
  GemmArgs a = make_args(A, K, a_panel, M, N, K);
  a.B.p[0] = B;
  a.ldb = K;
  if (out_dtype == TSP_BF16) {
    if (dtype != TSP_BF16) return hipErrorInvalidValue;
    EpiStoreBf16 e{(bf16 *)out, N};
    return run_gemm(dtype, a, e, s);
  }
  EpiStoreF32 e{(float *)out, N};
  return run_gemm(dtype, a, e, s);
}

}  // namespace tsp
