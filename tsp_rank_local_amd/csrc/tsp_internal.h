// Internal interface between the C-ABI layer (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tsp.h"

namespace tsp {

// Global position of local row t under the zigzag ownership of rank r:
// chunk r holds rows [0, C), chunk 2D-1-r holds rows [C, 2C).
struct ZigzagMap {
  int32_t C;      // chunk length S/(2D)
  int32_t base0;  // r*C
  int32_t base1;  // (2D-1-r)*C
  __host__ __device__ inline int32_t pos(int32_t t) const {
    return t < C ? base0 + t : base1 + (t - C);
  }
};

inline ZigzagMap make_zigzag(int64_t S, int32_t D, int32_t r) {
  ZigzagMap z;
  z.C = (int32_t)(S / (2 * D));
  z.base0 = r * z.C;
  z.base1 = (2 * D - 1 - r) * z.C;
  return z;
}

// Panel layout of the bf16 activations that feed a GEMM as its A operand
// (workspace tensors only): element (r, c) of an [M][K] tensor sits at
// (c / 64) * (M * 64) + r * 64 + c % 64, i.e. K is cut into panels of 64
// columns, each [M][64] row-major. A 256 x 64 GEMM tile is then 32 KB of
// contiguous memory. panel_stride = M * 64 elements; 0 means row-major.
constexpr int kPanel = 64;
__host__ __device__ inline int64_t panel_index(int64_t r, int64_t c, int64_t panel_stride) {
  return (c / kPanel) * panel_stride + r * kPanel + (c % kPanel);
}

// Up to TSP_MAX_D device pointers passed by value as a kernel argument.
struct PtrList {
  const void *p[TSP_MAX_D];
};

// ---------------------------------------------------------------- rows
hipError_t launch_zigzag_index(ZigzagMap zz, int32_t n, int32_t *pos, hipStream_t s);
// out[row] = x[row] / sqrt(mean(x[row]^2) + eps) * g, x fp32; g and out in
// dtype; out in panel layout when out_panel (panel stride rows * 64), else
// row-major.
hipError_t launch_rmsnorm(const float *x, const void *g, void *out, int32_t rows, int32_t h, float eps,
                          int dtype, bool out_panel, hipStream_t s);

// Same with fp32 output (row-major) and g in g_dtype.
hipError_t launch_rmsnorm_f32(const float *x, const void *g, int g_dtype, float *out, int32_t rows, int32_t h,
                              float eps, hipStream_t s);

// Backward of launch_rmsnorm for rows of x [rows][h] fp32 (h a multiple of 4,
// at most 8192) and output gradient d [rows][h] fp32: dx = (res ? res : 0) +
// the RMSNorm input gradient, fp32 [rows][h]; lo (optional) receives dx in
// dtype as well, in panel layout when lo_panel (bf16). dg [h] fp32 receives
// the gain gradient summed over the rows, through part (rmsnorm_bwd_part_bytes
// of scratch) in a fixed order. g in dtype.
size_t rmsnorm_bwd_part_bytes(int32_t rows, int32_t h);
hipError_t launch_rmsnorm_bwd(const float *x, const void *g, const float *d, const float *res, float *dx, void *lo,
                              bool lo_panel, int32_t rows, int32_t h, float eps, int dtype, float *part, float *dg,
                              hipStream_t s);
// out [n][D (wa + 2 wb)] in dtype (bf16 panel layout when out_panel): shard
// j's columns are a's columns j*wa.., then b's j*wb.., then c's j*wb.. (fp32
// sources [n][D wa] and [n][D wb]); wa, wb multiples of 4. D = 1, wb = 0
// converts a alone.
hipError_t launch_pack_cols(int dtype, const float *a, const float *b, const float *c, int32_t n, int32_t D,
                            int32_t wa, int32_t wb, void *out, bool out_panel, hipStream_t s);

// Rotary embedding (optional): table[t][i] = (cos, sin) of pos(t) *
// base^(-2i/Dh) for local rows t < n, pairs i < Dh/2 (computed in fp64).
hipError_t launch_rope_table(ZigzagMap zz, int32_t n, int32_t Dh, float base, float2 *table, hipStream_t s);
// In place on fp32 rows: row t at x + (scatter ? pos(t) : t) * ld holds H
// heads of Dh; pair i of each head (features i, i + Dh/2) turns by table[t][i].
hipError_t launch_rope_rows(float *x, int64_t ld, int32_t n, int32_t H, int32_t Dh, ZigzagMap zz, bool scatter,
                            const float2 *table, hipStream_t s);

// out(c, r) = in(r, c) for nz R x C matrices: matrix z is in.p[z] (row
// pitch in_ld, or panel layout with panel stride in_panel) and lands at
// out + z * out_zoff (row pitch out_ld, or panel layout with panel stride
// out_panel). Panel layouts are bf16 only.
hipError_t launch_transpose(int dtype, const PtrList &in, int32_t nz, int64_t in_ld, int64_t in_panel, int32_t R,
                            int32_t C, void *out, int64_t out_ld, int64_t out_panel, int64_t out_zoff, hipStream_t s);

// Z [n][F] bf16 (row-major) to Z^T in panel layout (panel stride F * 64) and
// GELU(Z)^T [F][n] row-major, in one pass (n and F multiples of 8).
hipError_t launch_transpose_gelu(const void *z, int32_t n, int32_t F, void *zt_panel, void *ht, hipStream_t s);

// ---------------------------------------------------------------- GEMMs
// All products are C = A B^T with A [M][K] and B [N][K] (both K-contiguous).
// a_panel: A in panel layout (bf16 only; panel stride M * 64), else row-major.
// QKV of every attention shard in one launch: shard z reads w[z]
// [hq + 2hk][h] (hq Q rows, hk K rows, hk V rows); Q columns go to q
// [n][D*hq] at column z*hq (multiplied by q_scale before rounding), K/V rows
// go to kf/vf [S][D*hk] at row zz.pos(t), column z*hk.
// rope (bf16 only, hq and hk multiples of 128): when not null, Q and K are
// rotated with the table of launch_rope_table (heads of Dh) before rounding.
hipError_t launch_qkv(int dtype, const void *xn, bool a_panel, int32_t n, int32_t h, const PtrList &w, int32_t D,
                      int32_t hq, int32_t hk, void *q, void *kf, void *vf, ZigzagMap zz, float q_scale,
                      const float2 *rope, int32_t Dh, hipStream_t s);
// y = x + sum_j o[:, j*hd:(j+1)*hd] wo[j]^T, shards walked j = 0..D-1 inside
// the reduction loop.
hipError_t launch_outproj(int dtype, const void *o, bool a_panel, int32_t n, int32_t h, const PtrList &wo,
                          int32_t D, int32_t hd, const float *x, float *y, hipStream_t s);
// MLP up over all D ring steps in one launch: hid[:, t*fd:(t+1)*fd] =
// GELU(x w1[t]^T) in dtype, w1[t] [fd][h] the shard of ring step t; hid
// [n][D*fd] (panel layout when hid_panel). gated: w1[t] is [2fd][h] (gate
// rows, then up rows) and hid = SiLU(x W_g^T) * (x W_u^T).
// z_out (bf16, GELU MLP only; else null): also write Z = x w1[t]^T before
// the GELU, [n][D*fd] row-major in the same column order as hid.
hipError_t launch_mlp_up(int dtype, const void *x, bool a_panel, int32_t n, int32_t h, const PtrList &w1, int32_t D,
                         int32_t fd, bool gated, void *hid, bool hid_panel, hipStream_t s, void *z_out = nullptr);
// y = (res ? res : 0) + sum_t hid[:, t*fd:(t+1)*fd] w2[t]^T in fp32, the
// reduction walking ring steps t = 0..D-1 in order; w2[t] [h][fd]; res may
// equal y.
hipError_t launch_mlp_down(int dtype, const void *hid, bool a_panel, int32_t n, const PtrList &w2, int32_t D,
                           int32_t fd, int32_t h, const float *res, float *y, hipStream_t s);

// MLP backward products (the MLP ring's gradients on one rank). The
// hidden-unit axis F is in ring-step order throughout (ring step t owns
// units t*fd..(t+1)*fd-1). zt_panel: Z^T / dZ^T [F][n] in panel layout
// (bf16 only, panel stride F * 64), else row-major with pitch n.
// Z^T = w1cat x^T (w1cat [F][h], x [n][h]): zt = Z^T, ht [F][n] row-major =
// GELU(Z^T), both in dtype.
hipError_t launch_mlp_bwd_recompute(int dtype, const void *w1cat, int32_t F, int32_t h, const void *x, int32_t n,
                                    void *zt, bool zt_panel, void *ht, hipStream_t s);
// dZ^T = (w2t dy^T) * GELU'(Z^T) (w2t [F][h], dy [n][h]), written over zt.
hipError_t launch_mlp_bwd_dz(int dtype, const void *w2t, int32_t F, int32_t h, const void *dy, int32_t n, void *zt,
                             bool zt_panel, hipStream_t s);
// Weight gradients over K = n tokens: C [M][N] = A [M][n] B [N][n]^T in
// fp32, A in panel layout when a_panel (bf16). by_rows: row m goes to
// out.p[m / split] row m % split (pitch N); else column c goes to
// out.p[c / split] column c % split (pitch split).
hipError_t launch_wgrad(int dtype, const void *a, bool a_panel, int32_t M, const void *b, int32_t N, int32_t n,
                        const PtrList &out, int32_t split, bool by_rows, hipStream_t s);
// dx = (res ? res : 0) + dz w1t^T: dz [n][F] (panel when a_panel), w1t [h][F].
hipError_t launch_mlp_bwd_dx(int dtype, const void *dz, bool a_panel, int32_t n, int32_t F, const void *w1t,
                             int32_t h, const float *res, float *dx, hipStream_t s);

// Plain product out [M][N] = A [M][K] B [N][K]^T (A in panel layout when
// a_panel), out row-major in out_dtype (bf16 only with bf16 operands).
hipError_t launch_gemm_nt(int dtype, const void *A, bool a_panel, int32_t M, int32_t K, const void *B, int32_t N,
                          void *out, int out_dtype, hipStream_t s);

// Leading rows in fp32: the same products for m <= kLeadRows rows with fp32
// activations (row-major) and the bf16 weights, computed to fp32 accuracy.
// part: scratch of lead_part_bytes(m, h, F, D) bytes (enough for any
// hk <= hq). QKV writes fp32 q [m][D*hq] and k/v rows zz.pos(t) of
// [*][D*hk] buffers (no Q factor).
constexpr int32_t kLeadRows = 64;
size_t lead_part_bytes(int32_t m, int32_t h, int32_t F, int32_t D, bool gated);
hipError_t launch_lead_qkv(const float *a, int32_t m, int32_t h, const PtrList &w, int32_t D, int32_t hq, int32_t hk,
                           float *q, float *k, float *v, ZigzagMap zz, float *part, hipStream_t s);
hipError_t launch_lead_outproj(const float *o, int32_t m, int32_t h, const PtrList &wo, int32_t D, int32_t hd,
                               const float *x, float *y, float *part, hipStream_t s);
hipError_t launch_lead_mlp_up(const float *a, int32_t m, int32_t h, const PtrList &w1, int32_t D, int32_t fd,
                              bool gated, float *hid, float *part, hipStream_t s);
hipError_t launch_lead_mlp_down(const float *hid, int32_t m, const PtrList &w2, int32_t D, int32_t fd, int32_t h,
                                const float *res, float *y, float *part, hipStream_t s);

// ---------------------------------------------------------------- attention
// q: [n][H][Dh]; k, v: [S][Hkv][Dh], query head i reading K/V head
// i / (H / Hkv) (H % Hkv == 0). o: [n][H][Dh] in o_dtype, or (bf16 o only)
// panel layout of [n][H*Dh] when o_panel. q_prescaled (bf16 q and o only): q
// already holds q * scale * log2(e), as launch_qkv writes it with that
// q_scale.
// lse (bf16 inputs, fp32 o; else null): also write each row's natural
// log-sum-exp of its scaled scores, [H][n] fp32 (with q_prescaled as well:
// the training forward of the layer).
hipError_t launch_attention(int dtype, const void *q, const void *k, const void *v, void *o, int o_dtype,
                            bool o_panel, int64_t S, int32_t n, int32_t H, int32_t Hkv, int32_t Dh, float scale,
                            ZigzagMap zz, bool q_prescaled, hipStream_t s, float *lse = nullptr);
// fp32 attention of the first m <= 64 positions among themselves (the
// leading rows of rank 0): q, o [m][H][Dh], k, v [m][Hkv][Dh] fp32, key j
// visible to query i when j <= i.
hipError_t launch_lead_attention(const float *q, const float *k, const float *v, float *o, int32_t m, int32_t H,
                                 int32_t Hkv, int32_t Dh, float scale, hipStream_t s);

// Backward of launch_attention (bf16 or fp32 inputs, no pre-scaled Q): q,
// dout [n][H][Dh] and k, v [S][Hkv][Dh] in dtype; dq [n][H][Dh] and the
// rank's contributions dk, dv [S][Hkv][Dh] in fp32 (every row written). lse,
// delta: scratch [H][n] fp32 each (log2-domain log-sum-exp of each row, and
// sum over its keys of P dP).
// With o_f32 and lse_in given (bf16 inputs; the forward's fp32 output and
// natural log-sum-exp [H][n] of launch_attention), Delta is the row sum of
// dout * o and the statistics walk of the dQ kernel is skipped.
// split (bf16): P and dS enter their products as a bf16 pair hi + lo;
// otherwise rounded once to bf16.
// q_prescaled (with o_f32 and lse_in only): q holds q * scale * log2(e) as
// the layer's QKV epilogue writes it (and lse_in came from the forward on
// that q); dq is still the gradient of the unscaled q.
hipError_t launch_attention_bwd(int dtype, const void *q, const void *k, const void *v, const void *dout, float *dq,
                                float *dk, float *dv, float *lse, float *delta, int64_t S, int32_t n, int32_t H,
                                int32_t Hkv, int32_t Dh, float scale, ZigzagMap zz, hipStream_t s,
                                const float *o_f32 = nullptr, const float *lse_in = nullptr, bool split = true,
                                bool q_prescaled = false);

// ---------------------------------------------------------------- static scratch
// Size of the device array that tsp_zigzag_attn_bwd_noalloc uses in place of
// a caller's workspace (one array per GPU, shared by every such call on it).
constexpr size_t kNoallocScratchBytes = size_t(8) << 20;
// Device address of that array on the stream's device (which must be the
// current device); looked up once per device and kept.
hipError_t noalloc_scratch(hipStream_t stream, void **addr);

// ---------------------------------------------------------------- timing
// Bracket a launch with events when profiling is on (api.cpp).
void prof_begin(int kclass, hipStream_t s);
void prof_end(int kclass, hipStream_t s);

}  // namespace tsp
