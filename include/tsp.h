/*
 * tsp.h - C ABI of the rank-local TSP decoder-layer forward for MI355X (gfx950).
 *
 * TSP ("folded" tensor + sequence parallelism) puts weight sharding and token
 * sharding on one device-mesh axis of size D: every rank keeps 1/D of each
 * weight matrix and 1/D of the sequence tokens (zubnet.ai news item "Zyphra
 * TSP folds TP+SP onto one GPU axis", paragraph 1). For attention the weight
 * shards are broadcast one after another and each rank applies every shard to
 * its own tokens, after which K and V are all-gathered under a zigzag
 * partition; for the MLP the weight shards circulate round a ring of
 * point-to-point transfers and each rank sums the shard contributions itself,
 * with no all-reduce (same page, paragraph 2; paragraph 4 notes that this MLP
 * scheme carries over to other setups).
 *
 * This library computes ONE rank's share of that forward pass on one GPU.
 * The shards that the broadcasts and the ring would deliver are passed as
 * arrays of D device pointers, and the K/V rows the all-gather would deliver
 * are caller-filled rows of full-sequence buffers. Nothing is communicated.
 *
 * Readings taken where the pages are silent:
 *  - zigzag: the sequence is cut into 2D chunks of C = S/(2D) tokens; rank r
 *    holds chunk r then chunk 2D-1-r, ascending inside each chunk, so local
 *    row t sits at global position  r*C + t  (t < C)  or  (2D-1-r)*C + t - C.
 *  - attention shard j is head group j: heads j*H/D .. (j+1)*H/D-1.
 *  - causal mask is inclusive (key u visible to query p iff u <= p); no bias,
 *    no rotary embedding; multi-head attention with H query and H K/V heads.
 *  - pre-RMSNorm block, eps from the shape: h1 = x + Attn(RMSNorm(x) g_attn),
 *    y = h1 + GELU(RMSNorm(h1) g_mlp W1^T) W2^T, exact (erf) GELU, no biases.
 *  - delivery order: attention shards j = 0..D-1 (broadcast roots in turn);
 *    MLP shard at ring step t is j = (r - t) mod D.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers unless marked (host). Row-major,
 *    innermost index last; every tensor pointer must be 16-byte aligned.
 *  - 'stream' is a hipStream_t passed as void* (NULL = default stream). All
 *    work is enqueued on it asynchronously; the call returns before it runs.
 *  - The caller owns every buffer; the library allocates no device memory and
 *    keeps no pointer after it returns (its only device memory of its own is
 *    the static scratch array of tsp_zigzag_attn_bwd_noalloc, 8 MiB per GPU,
 *    part of the loaded library). Buffers must stay valid until the enqueued
 *    work has finished.
 *  - dtype TSP_BF16: weights, gains, x of tsp_mlp_ring, Q/K/V, O and the MLP
 *    hidden activations are bf16; the residual stream x/h1/y of the layer is
 *    fp32; every product accumulates in fp32. In attention the probabilities
 *    enter the P.V product rounded to bf16, except in query tiles whose
 *    positions all lie below 1024, where they enter as a bf16 pair hi + lo
 *    (those rows see few keys, so a single weight can carry most of a row).
 *    dtype TSP_F32: everything is fp32.
 *  - Errors: all arguments are checked on the host before anything is
 *    enqueued. On failure nothing is enqueued, the status is returned and
 *    tsp_last_error() describes the problem (thread-local). TSP_ERR_HIP means
 *    a launch was rejected by the runtime; faults inside kernels surface at
 *    the caller's next stream synchronisation.
 *  - Results are deterministic: identical inputs give identical bits.
 */
#ifndef TSP_H
#define TSP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TSP_OK = 0,
  TSP_ERR_INVALID_ARG = 1, /* null/misaligned pointer, inconsistent shape, overlap */
  TSP_ERR_UNSUPPORTED = 2, /* valid but not handled: Dh not 64/128, widths not multiples of 64 */
  TSP_ERR_WORKSPACE = 3,   /* ws_bytes below tsp_workspace_size() */
  TSP_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} tsp_status;

typedef enum { TSP_F32 = 0, TSP_BF16 = 1 } tsp_dtype;

/* MLP form (tsp_shape.mlp).
 *  TSP_MLP_GELU:   GELU(x W1^T) W2^T, exact erf GELU (the pages' "FFN x4"
 *                  model, [P2] paragraph 1).
 *  TSP_MLP_SWIGLU: (SiLU(x Wg^T) * (x Wu^T)) W2^T, SiLU(z) = z / (1 + e^-z)
 *                  (an optional variant, the gated MLP of common 7B models;
 *                  not on the pages). Shard j's first matrix stacks its F/D
 *                  Wg rows on the Wu rows of the same hidden units. */
typedef enum { TSP_MLP_GELU = 0, TSP_MLP_SWIGLU = 1 } tsp_mlp_kind;

/* Sizes of one layer on the folded axis.
 *  S  total sequence length (the K/V all-gather covers S rows), S < 2^31
 *  D  axis size (number of ranks / shards), 1 <= D <= TSP_MAX_D, S % (2D) == 0
 *  r  this rank, 0 <= r < D
 *  h  hidden width, h == H*Dh;  H heads (H % D == 0 for the layer);  Dh 64 or 128
 *  F  MLP width, F % D == 0
 *  eps   RMSNorm epsilon (>= 0)
 *  scale softmax scale applied to q.k (finite, >= 0; usually 1/sqrt(Dh))
 *  dtype tsp_dtype of weights and activations (see conventions)
 *  rope_base rotary position embedding of Q and K in tsp_layer_fwd (an
 *        optional variant; the pages' model has none): 0 = none; > 0: within
 *        each head, features i and i + Dh/2 form pair i, which turns by the
 *        angle pos * rope_base^(-2i/Dh), pos = the token's global position.
 *        bf16 layers need h/D to be a multiple of 128 for it (else
 *        TSP_ERR_UNSUPPORTED). tsp_zigzag_attn takes Q and K as given.
 *  Hkv   K/V heads (grouped-query attention, an optional variant; the
 *        pages' model is multi-head): 0 = H. Otherwise Hkv divides H and
 *        query head i reads K/V head i / (H/Hkv); the layer also needs
 *        Hkv % D == 0, so head group j holds query heads j*H/D.. and K/V
 *        heads j*Hkv/D.., and bf16 rotation needs Hkv*Dh/D % 128 == 0.
 *  mlp   tsp_mlp_kind of tsp_mlp_ring and tsp_layer_fwd (0 = GELU, the
 *        pages' model). F is the number of hidden units either way.
 * Local token count N = S/D. Widths used as GEMM dimensions (h, F/D, h/D)
 * must be multiples of 64. */
typedef struct {
  int64_t S;
  int32_t D, r, h, H, Dh, F;
  float eps, scale;
  int32_t dtype;
  float rope_base;
  int32_t Hkv;
  int32_t mlp;
} tsp_shape;

#define TSP_MAX_D 64

/* One layer's weights. The four shard arrays are (host) arrays of D device
 * pointers indexed by SHARD id j (not by delivery step); matrices are stored
 * (out, in), so every product reads its operands along the contiguous axis.
 *  g_attn, g_mlp: [h] RMSNorm gains (dtype).
 *  wqkv[j]: [(H + 2Hkv)Dh/D][h]  rows: the Q rows of head group j (H/D
 *           heads), then its K rows, then its V rows (Hkv/D heads each),
 *           each head-major (head, then feature within the head).
 *  wo[j]:   [h][h/D]   the columns of W_O that read head group j.
 *  w1[j]:   [F/D][h]   rows j*F/D.. of W1; TSP_MLP_SWIGLU: [2F/D][h], rows
 *           j*F/D.. of Wg, then the same rows of Wu.
 *  w2[j]:   [h][F/D]   columns j*F/D.. of W2. */
typedef struct {
  const void *g_attn;
  const void *g_mlp;
  const void *const *wqkv;
  const void *const *wo;
  const void *const *w1;
  const void *const *w2;
} tsp_layer_weights;

/* Phases of tsp_layer_fwd, for emulating the K/V all-gather of several ranks
 * on one GPU: PHASE_KV runs RMSNorm-1 and the QKV shards, writes this rank's
 * K/V rows into k_full/v_full and keeps Q in the workspace; PHASE_REST runs
 * attention, the output projection and the MLP ring from that workspace. */
enum { TSP_PHASE_KV = 1, TSP_PHASE_REST = 2, TSP_PHASE_ALL = 3 };

/* Workspace kinds for tsp_workspace_size. */
enum { TSP_WS_MLP = 0, TSP_WS_LAYER = 1, TSP_WS_MLP_BWD = 2, TSP_WS_ATTN_BWD = 3, TSP_WS_LAYER_BWD = 4 };

/* Phases of tsp_layer_bwd: the two halves of a rank's layer backward on
 * either side of the exchange that returns key/value gradients to the ranks
 * that own those rows. */
enum { TSP_BWD_ATTN = 1, TSP_BWD_QKV = 2, TSP_BWD_ALL = 3 };

/* Gradients of one layer's weights, laid out as tsp_layer_weights, fp32:
 * g_attn, g_mlp [h]; wqkv, wo, w1, w2 (host) arrays of D device pointers with
 * the shard shapes of tsp_layer_weights. */
typedef struct {
  float *g_attn;
  float *g_mlp;
  float *const *wqkv;
  float *const *wo;
  float *const *w1;
  float *const *w2;
} tsp_layer_grads;

/* Kernel classes for the optional launch timing. */
enum {
  TSP_K_RMSNORM = 0,
  TSP_K_QKV = 1,
  TSP_K_ATTN = 2,
  TSP_K_OUTPROJ = 3,
  TSP_K_MLP_UP = 4,
  TSP_K_MLP_DOWN = 5,
  TSP_K_ZIGZAG = 6,
  TSP_K_LEAD = 7, /* the fp32 recomputation of the leading rows (see tsp_layer_fwd) */
  TSP_K_BWD_GEMM = 8,  /* the products of tsp_mlp_ring_bwd */
  TSP_K_TRANSPOSE = 9, /* the layout changes of tsp_mlp_ring_bwd */
  TSP_K_ATTN_BWD = 10, /* the launches of tsp_zigzag_attn_bwd */
  TSP_K_ROWS_BWD = 11, /* the RMSNorm backward and column packing of tsp_layer_bwd */
  TSP_K_COUNT = 12
};

/* Static text for a status code. */
const char *tsp_status_string(int status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char *tsp_last_error(void);

/* ABI version of this header (bumped on incompatible change). */
int tsp_abi_version(void);

/* Bytes of scratch the call 'which' (TSP_WS_MLP for tsp_mlp_ring,
 * TSP_WS_LAYER for tsp_layer_fwd, TSP_WS_MLP_BWD for tsp_mlp_ring_bwd,
 * TSP_WS_ATTN_BWD for tsp_zigzag_attn_bwd, TSP_WS_LAYER_BWD for
 * tsp_layer_bwd) needs for this shape. */
tsp_status tsp_workspace_size(const tsp_shape *shape, int which, size_t *bytes);

/* Zigzag token ownership (reading above; the pages name a zigzag partition
 * for load balance, paragraph 2): pos[t] = global position of local row t,
 * t < S/D. _host fills a (host) array; the other form launches a kernel that
 * fills a device int32 array on 'stream'. Both give identical values. */
tsp_status tsp_zigzag_index_host(int64_t S, int32_t D, int32_t r, int32_t *pos);
tsp_status tsp_zigzag_index(int64_t S, int32_t D, int32_t r, int32_t *pos, void *stream);

/* Causal attention of rank r's local queries against the gathered K/V
 * (paragraph 2: K/V are all-gathered, so every rank sees the full sequence).
 *  q: [S/D][H][Dh] local rows in zigzag order (dtype)
 *  k, v: [S][Hkv][Dh] all positions in global order (dtype)
 *  o: [S/D][H][Dh] output (o_dtype: TSP_F32, or TSP_BF16 when dtype is bf16)
 * o[t][i] = sum_{u <= pos[t]} softmax_u(scale * q[t][i].k[u][j]) v[u][j],
 * j = i / (H/Hkv) (j = i when Hkv is 0 or H).
 * Uses S, D, r, H, Hkv, Dh, scale and dtype of the shape. */
tsp_status tsp_zigzag_attn(const tsp_shape *shape, const void *q, const void *k, const void *v,
                           void *o, int32_t o_dtype, void *stream);

/* Flags of tsp_zigzag_attn_ex. */
enum { TSP_ATTN_Q_LOG2_SCALED = 1 };

/* tsp_zigzag_attn with flags (0 gives tsp_zigzag_attn).
 *  TSP_ATTN_Q_LOG2_SCALED: q holds q * scale * log2(e), as a caller that folds
 *    the softmax scale into its Q projection would store it (the layer does
 *    this); the result is the same attention, with one fewer multiply per
 *    score. bf16 q and o only (else TSP_ERR_UNSUPPORTED). Unknown flag bits
 *    are TSP_ERR_INVALID_ARG. */
tsp_status tsp_zigzag_attn_ex(const tsp_shape *shape, const void *q, const void *k, const void *v,
                              void *o, int32_t o_dtype, uint32_t flags, void *stream);

/* The MLP ring on rank r (paragraph 2: shards circulate on a ring and every
 * rank sums their contributions itself, with no all-reduce):
 *   y = residual + sum over steps t = 0..D-1 of GELU(x W1_j^T) W2_j^T,
 *   j = (r - t) mod D, accumulated into y in fp32 in that order (with
 *   TSP_MLP_SWIGLU the hidden layer is SiLU(x Wg_j^T) * (x Wu_j^T)).
 *  x: [S/D][h] (dtype); w1, w2: (host) arrays of D device pointers, shard
 *  layout as in tsp_layer_weights; residual: [S/D][h] fp32 or NULL (then
 *  zero); it may equal y. y: [S/D][h] fp32, fully written.
 *  ws: device scratch of at least tsp_workspace_size(TSP_WS_MLP) bytes. */
tsp_status tsp_mlp_ring(const tsp_shape *shape, const void *x, const void *const *w1,
                        const void *const *w2, const float *residual, float *y, void *ws,
                        size_t ws_bytes, void *stream);

/* Backward of the zigzag causal attention on rank r (an optional extension,
 * like tsp_mlp_ring_bwd: the pages give no backward). For the forward of
 * tsp_zigzag_attn, o = softmax(scale q k^T, causal) v over the gathered K/V,
 * and an output gradient dout, with p the probabilities, dp = dout v^T and
 * ds = p * (dp - sum over the row's keys of p dp) (the softmax Jacobian; the
 * sum equals rowsum(dout * o) and is formed from the fp32 probabilities, so
 * the forward's output is not needed):
 *   dq = scale ds k           [S/D][H][Dh]  this rank's queries;
 *   dk = scale ds^T q,  dv = p^T dout   [S][Hkv][Dh]  this rank's queries'
 *   contribution to every key and value row (zero past the rank's last
 *   position; the D ranks' contributions add up to the gradients over the
 *   whole sequence, which would travel back to each row's owner).
 *  q, dout: [S/D][H][Dh] (dtype), local rows in zigzag order, q unscaled;
 *  k, v: [S][Hkv][Dh] (dtype), global order. dq, dk, dv: fp32, fully
 *  written. Rounding (bf16): p enters p^T dout and ds enters ds k and ds^T q
 *  as a bf16 pair hi + lo (exact to about 2^-16 of their size); row
 *  statistics, dp, ds and all accumulation are fp32.
 *  ws: device scratch of at least tsp_workspace_size(TSP_WS_ATTN_BWD) bytes. */
tsp_status tsp_zigzag_attn_bwd(const tsp_shape *shape, const void *q, const void *k, const void *v,
                               const void *dout, float *dq, float *dk, float *dv, void *ws,
                               size_t ws_bytes, void *stream);

/* tsp_zigzag_attn_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, arguments and errors, but the row
 * statistics live in a static device array of the library (8 MiB per GPU,
 * reserved from the library's load until the process ends) instead of a
 * caller's workspace; it allocates nothing. Limit: H * S/D <= 1048576 (the
 * 7B shape at 128K tokens and D = 8 uses half); larger shapes return
 * TSP_ERR_UNSUPPORTED with nothing enqueued. The stream's device must be
 * the current device (else TSP_ERR_INVALID_ARG). All calls on one GPU share
 * its array, and each call writes every entry it later reads, so nothing
 * carries over between calls; calls that overlap in time on one GPU (two
 * streams, two threads) race on it and must be serialised by the caller. */
tsp_status tsp_zigzag_attn_bwd_noalloc(const tsp_shape *shape, const void *q, const void *k, const void *v,
                                       const void *dout, float *dq, float *dk, float *dv, void *stream);

/* Flags of tsp_zigzag_attn_bwd_ex. */
enum { TSP_ATTN_BWD_PLAIN_PDS = 1 };

/* tsp_zigzag_attn_bwd with flags, and with the forward's statistics
 * optional: o and lse both NULL (the kernels take the row statistics
 * themselves, as tsp_zigzag_attn_bwd) or both given (as
 * tsp_zigzag_attn_bwd_lse, bf16 only). TSP_ATTN_BWD_PLAIN_PDS (bf16 inputs,
 * else TSP_ERR_UNSUPPORTED): P and dS enter their products rounded once to
 * bf16, one matrix product each, instead of as the hi + lo pair; this saves
 * a third of the matrix products and most of the conversions. The error is
 * then that of common flash-attention backward kernels: norm-wise about the
 * bf16 rounding unit, but single elements of the largest gradient rows can
 * be off by several percent of the tensor's rms. tsp_layer_bwd uses it.
 * Unknown flags: TSP_ERR_INVALID_ARG. Otherwise as tsp_zigzag_attn_bwd. */
tsp_status tsp_zigzag_attn_bwd_ex(const tsp_shape *shape, const void *q, const void *k, const void *v,
                                  const float *o, const float *lse, const void *dout, float *dq, float *dk,
                                  float *dv, uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* tsp_zigzag_attn for the backward's use: bf16 inputs (else
 * TSP_ERR_UNSUPPORTED), plain q, o in fp32 [S/D][H][Dh], and also lse
 * [H][S/D] fp32, the natural log of each row's softmax denominator,
 * log sum_u exp(scale q.k_u) over its visible keys. Errors as for
 * tsp_zigzag_attn; o and lse must not overlap the inputs or each other. */
tsp_status tsp_zigzag_attn_lse(const tsp_shape *shape, const void *q, const void *k, const void *v,
                               float *o, float *lse, void *stream);

/* tsp_zigzag_attn_bwd with the row statistics of the forward (bf16 inputs,
 * else TSP_ERR_UNSUPPORTED): o and lse are the outputs of
 * tsp_zigzag_attn_lse for the same q, k, v. Each row's sum over its keys of
 * p dp is then taken as rowsum(dout * o) from the fp32 o, and p from lse,
 * which saves the kernels one pass over the keys; everything else is as in
 * tsp_zigzag_attn_bwd (same workspace). */
tsp_status tsp_zigzag_attn_bwd_lse(const tsp_shape *shape, const void *q, const void *k, const void *v,
                                   const float *o, const float *lse, const void *dout, float *dq,
                                   float *dk, float *dv, void *ws, size_t ws_bytes, void *stream);

/* Backward of the MLP ring on rank r (an optional extension: the pages quote
 * their 2.6x for training, [P2] paragraph 1, but describe only how the
 * shards move, paragraph 2). With Z = x W1^T and y = GELU(Z) W2^T summed over
 * the shards, and dy the gradient of y:
 *   dx     = dx_residual + sum over ring steps t of (dy W2_j * GELU'(Z_j)) W1_j,
 *            j = (r - t) mod D, reduced in fp32 in that order (again with no
 *            all-reduce: every rank sums the shards it receives itself);
 *   dw1[j] = dZ_j^T x   [F/D][h],  dZ_j = (dy W2_j) * GELU'(Z_j);
 *   dw2[j] = dy^T GELU(Z_j)   [h][F/D];
 * the weight gradients being this rank's own tokens' contribution (the D
 * ranks' contributions add up to the shard's gradient over the sequence, the
 * sum a ring would carry back to the shard's owner). GELU MLP only
 * (tsp_shape.mlp = TSP_MLP_GELU, else TSP_ERR_UNSUPPORTED); S/D must be a
 * multiple of 64.
 *  x, dy: [S/D][h] (dtype), the branch input of tsp_mlp_ring and the gradient
 *  of its output; w1, w2: (host) arrays of D device pointers, shard layout as
 *  in tsp_layer_weights. dx_residual: [S/D][h] fp32 or NULL (then zero); it
 *  may equal dx. dx: [S/D][h] fp32, dw1/dw2: (host) arrays of D device
 *  pointers to fp32 buffers, all fully written. Z is recomputed (Z and
 *  GELU(Z) rounded to dtype once, as the forward stores GELU(Z)); dZ is
 *  rounded to dtype once; every product accumulates in fp32.
 *  ws: device scratch of at least tsp_workspace_size(TSP_WS_MLP_BWD) bytes. */
tsp_status tsp_mlp_ring_bwd(const tsp_shape *shape, const void *x, const void *const *w1,
                            const void *const *w2, const void *dy, const float *dx_residual,
                            float *dx, float *const *dw1, float *const *dw2, void *ws,
                            size_t ws_bytes, void *stream);

/* tsp_mlp_ring that also keeps the pre-activation for the backward (bf16,
 * GELU MLP only, else TSP_ERR_UNSUPPORTED): z [S/D][F] bf16 receives
 * Z = x W1_j^T of every ring step t in columns t*F/D.., rounded once from the
 * fp32 product; z must not overlap x, y, residual or ws. */
tsp_status tsp_mlp_ring_z(const tsp_shape *shape, const void *x, const void *const *w1,
                          const void *const *w2, const float *residual, float *y, void *z, void *ws,
                          size_t ws_bytes, void *stream);

/* tsp_mlp_ring_bwd with the pre-activation given (bf16 only): z is the z of
 * tsp_mlp_ring_z for the same shape (same r, so the same column order) and
 * x. Z is then not recomputed; GELU(Z) for dW2 is taken from the bf16 Z.
 * Everything else is as in tsp_mlp_ring_bwd (same workspace). */
tsp_status tsp_mlp_ring_bwd_z(const tsp_shape *shape, const void *x, const void *z,
                              const void *const *w1, const void *const *w2, const void *dy,
                              const float *dx_residual, float *dx, float *const *dw1,
                              float *const *dw2, void *ws, size_t ws_bytes, void *stream);

/* One decoder layer forward on rank r's S/D tokens: the whole folded-axis
 * schedule of the zubnet.ai news item "Zyphra TSP folds TP+SP onto one GPU
 * axis" on one rank. Paragraph 1: the rank holds 1/D of the tokens and 1/D
 * of every weight matrix. Paragraph 2: the attention weight shards arrive by
 * broadcast, one after another, and the rank applies each to its own tokens
 * (QKV, then the output projection); K and V are all-gathered under the
 * zigzag partition before attention; the MLP shards arrive round a ring and
 * the rank sums their contributions itself, with no all-reduce.
 *  x: [S/D][h] fp32, local rows in zigzag order.
 *  k_full, v_full: [S][Hkv][Dh] (dtype). The rows at rank r's own positions are
 *    written by PHASE_KV; every other row must hold what the all-gather would
 *    deliver (the other ranks' K/V, K already rotated when rope_base > 0)
 *    before PHASE_REST runs.
 *  y: [S/D][h] fp32 output, fully written by PHASE_REST.
 *  phases: TSP_PHASE_KV, TSP_PHASE_REST or TSP_PHASE_ALL; PHASE_REST must use
 *    the same ws as the PHASE_KV call before it.
 *  ws: device scratch of at least tsp_workspace_size(TSP_WS_LAYER) bytes.
 * y must not overlap x, k_full, v_full or ws.
 * bf16 rank 0: the queries at positions below min(64, S/(2D)) attend to so
 * few keys that their output is not averaged down, and the bf16 storage of
 * the intermediates (normed input, Q/K/V, attention output, MLP input and
 * hidden layer) alone brings their error close to 2e-2 of the output rms.
 * PHASE_REST therefore recomputes those rows, which see only each other, with
 * fp32 intermediates and fp32-accurate products (the bf16 weights are exact),
 * and writes their y from that; their K/V rows in k_full/v_full stay bf16. */
tsp_status tsp_layer_fwd(const tsp_shape *shape, const tsp_layer_weights *w, const float *x,
                         void *k_full, void *v_full, float *y, unsigned phases, void *ws,
                         size_t ws_bytes, void *stream);

/* tsp_layer_fwd for training: the same layer (the passages and arguments
 * above, y the same bit for bit), and in the same pass the attention output
 * and its rows' statistics, kept for tsp_layer_bwd_ex so that the backward
 * does not run the attention forward again (the pages report training
 * throughput: the ageofai.tools review "Zyphra TSP: 2.6x Faster AI Training
 * Review", key features and benefits). bf16 only (else
 * TSP_ERR_UNSUPPORTED).
 *  o_save: [S/D][H][Dh] fp32, the attention output O before the output
 *    projection (which reads it rounded to bf16), written by PHASE_REST. On
 *    rank 0 the first rows are those of the bf16 path (their y is
 *    recomputed in fp32 as above, their O is not).
 *  lse_save: [H][S/D] fp32, each row's natural log-sum-exp of its scaled
 *    scores (over its visible keys), written by PHASE_REST.
 *  z_save: optional (NULL: not kept), [S/D][F] bf16, the MLP pre-activation
 *    Z of every ring step (as tsp_mlp_ring_z writes it), written by
 *    PHASE_REST; GELU MLP only (else TSP_ERR_UNSUPPORTED).
 * o_save and lse_save must both be given; none may overlap any other
 * argument. */
tsp_status tsp_layer_fwd_save(const tsp_shape *shape, const tsp_layer_weights *w, const float *x,
                              void *k_full, void *v_full, float *y, float *o_save, float *lse_save,
                              void *z_save, unsigned phases, void *ws, size_t ws_bytes, void *stream);

/* Backward of tsp_layer_fwd on rank r (an optional extension, like
 * tsp_mlp_ring_bwd: the pages report training throughput, the ageofai.tools
 * review "Zyphra TSP: 2.6x Faster AI Training Review", key features and
 * benefits, but describe no backward). It keeps the forward's schedule (the
 * zubnet.ai news item, paragraph 2): the rank applies the weight shards it
 * receives to its own tokens and sums the MLP ring's contributions itself;
 * the only new exchange is the reverse of the K/V all-gather, a
 * reduce-scatter that returns each key/value row's gradient to its owner,
 * between the two phases. Chain rule on the pre-norm layer, forward
 * recomputed from x:
 *  TSP_BWD_ATTN: xn = RMSNorm(x) g_attn, Q, attention (o, and its row
 *    statistics), h1 = x + o W_O^T, hn = RMSNorm(h1) g_mlp; then the MLP
 *    ring backward of tsp_mlp_ring_bwd on hn and dy, the second RMSNorm's
 *    backward, dh1 = dy + that; do = dh1 W_O, dW_O = dh1^T o; the attention
 *    backward of tsp_zigzag_attn_bwd_ex (the forward's statistics given,
 *    TSP_ATTN_BWD_PLAIN_PDS), giving dq (kept in ws) and this rank's
 *    contribution dk_full, dv_full to every key/value row.
 *  TSP_BWD_QKV, once dk_loc, dv_loc hold the summed gradients of the rank's
 *    own K/V rows: dxn = [dq | dk | dv] W_QKV over the shards,
 *    dW_QKV,j = [dq_j | dk_j | dv_j]^T xn, and dx = dh1 + the first
 *    RMSNorm's backward of dxn.
 * Weight and gain gradients are this rank's tokens' contribution (the D
 * ranks' contributions add up to the gradient over the whole sequence).
 * Supported: GELU MLP, no rotary embedding, S/D a multiple of 64, h <= 8192
 * (else TSP_ERR_UNSUPPORTED, nothing enqueued).
 *  x, dy: [S/D][h] fp32, local rows in zigzag order (dy: gradient of y).
 *  k_full, v_full: [S][Hkv][Dh] (dtype), the gathered K/V of the forward.
 *  dk_full, dv_full: [S][Hkv][Dh] fp32, fully written by TSP_BWD_ATTN.
 *  dk_loc, dv_loc: [S/D][Hkv][Dh] fp32, read by TSP_BWD_QKV: row t is the
 *    gradient of the K/V row at the rank's position pos(t), summed over the
 *    D ranks. With D = 1 they may be dk_full and dv_full themselves, and
 *    TSP_BWD_ALL runs both phases in one call (D = 1 only).
 *  dx: [S/D][h] fp32, written by TSP_BWD_QKV.
 *  grads: written: wo, w1, w2, g_mlp by TSP_BWD_ATTN; wqkv, g_attn by
 *    TSP_BWD_QKV. Pointers a phase does not touch may be NULL.
 *  ws: device scratch of at least tsp_workspace_size(TSP_WS_LAYER_BWD)
 *    bytes; TSP_BWD_QKV reads what TSP_BWD_ATTN left there (dh1 and dq),
 *    so both phases use the same ws.
 * Rounding (bf16): xn, Q, o (for the products), hn, dy (for the MLP
 * products), dh1 (for its products), do, the attention's P and dS, and
 * dq/dk/dv (for the QKV products) are rounded once to bf16; RMSNorm
 * statistics, the residual-stream gradients dh1 and dx and all
 * accumulation are fp32. Outputs must not
 * overlap inputs or each other. */
tsp_status tsp_layer_bwd(const tsp_shape *shape, const tsp_layer_weights *w, const float *x,
                         const void *k_full, const void *v_full, const float *dy, float *dk_full,
                         float *dv_full, const float *dk_loc, const float *dv_loc, float *dx,
                         const tsp_layer_grads *grads, unsigned phases, void *ws, size_t ws_bytes,
                         void *stream);

/* tsp_layer_bwd with the attention output and statistics that
 * tsp_layer_fwd_save kept (same passages and arguments as tsp_layer_bwd).
 * o_saved [S/D][H][Dh] and lse_saved [H][S/D] fp32, both NULL (then the call
 * is tsp_layer_bwd) or both given (bf16 only, else TSP_ERR_UNSUPPORTED;
 * read by TSP_BWD_ATTN): the attention forward is not run again. Q is
 * recomputed with the forward's pre-scaling by scale * log2(e), which
 * reproduces the forward's Q bit for bit, so the saved statistics belong to
 * the scores the backward forms; dK is then ln 2 * dS^T Q' (Q' the
 * pre-scaled Q), the same gradient. z_saved (optional, with o_saved and
 * lse_saved; tsp_layer_fwd_save's z_save): the MLP ring backward then takes
 * Z as tsp_mlp_ring_bwd_z does instead of recomputing it. They must come from
 * the forward of the same x, weights and K/V. */
tsp_status tsp_layer_bwd_ex(const tsp_shape *shape, const tsp_layer_weights *w, const float *x,
                            const void *k_full, const void *v_full, const float *dy,
                            const float *o_saved, const float *lse_saved, const void *z_saved,
                            float *dk_full, float *dv_full, const float *dk_loc, const float *dv_loc,
                            float *dx, const tsp_layer_grads *grads, unsigned phases, void *ws,
                            size_t ws_bytes, void *stream);

/* Optional launch timing. When enabled, every kernel the library enqueues is
 * bracketed by HIP events recorded on the same stream; tsp_profile_read
 * synchronises on the recorded events and returns the summed duration (ms)
 * and number of launches for one kernel class since the last reset. Not
 * thread-safe; meant for benchmarks. */
void tsp_profile_enable(int on);
void tsp_profile_reset(void);
tsp_status tsp_profile_read(int kernel_class, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* TSP_H */
