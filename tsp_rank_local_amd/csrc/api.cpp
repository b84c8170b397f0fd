// C ABI of the rank-local TSP layer: argument checks, workspace layout and the
// order of launches. Every check runs on the host before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "tsp_internal.h"

namespace {

thread_local std::string g_err;

tsp_status fail(tsp_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

tsp_status ok() {
  g_err.clear();
  return TSP_OK;
}

size_t elem_bytes(int dtype) { return dtype == TSP_BF16 ? 2 : 4; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void *p;
  size_t bytes;
  const char *name;
};

bool overlap(const Range &a, const Range &b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

tsp_status check_ptr(const void *p, const char *name) {
  if (!p) return fail(TSP_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(TSP_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return TSP_OK;
}

tsp_status check_ptr_list(const void *const *list, int D, const char *name) {
  if (!list) return fail(TSP_ERR_INVALID_ARG, "%s (array of shard pointers) is NULL", name);
  for (int j = 0; j < D; ++j) {
    if (!list[j]) return fail(TSP_ERR_INVALID_ARG, "%s[%d] is NULL", name, j);
    if (!aligned16(list[j])) return fail(TSP_ERR_INVALID_ARG, "%s[%d] is not 16-byte aligned", name, j);
  }
  return TSP_OK;
}

// Checks shared by every entry point: the folded axis and the zigzag split.
tsp_status check_axis(const tsp_shape *s) {
  if (!s) return fail(TSP_ERR_INVALID_ARG, "shape is NULL");
  if (s->D < 1 || s->D > TSP_MAX_D) return fail(TSP_ERR_INVALID_ARG, "D=%d outside [1, %d]", s->D, TSP_MAX_D);
  if (s->S <= 0 || s->S >= (int64_t(1) << 31)) return fail(TSP_ERR_INVALID_ARG, "S=%lld outside [1, 2^31)", (long long)s->S);
  if (s->S % (2 * s->D) != 0) return fail(TSP_ERR_INVALID_ARG, "S=%lld is not a multiple of 2D=%d", (long long)s->S, 2 * s->D);
  if (s->r < 0 || s->r >= s->D) return fail(TSP_ERR_INVALID_ARG, "r=%d outside [0, D=%d)", s->r, s->D);
  if (s->dtype != TSP_F32 && s->dtype != TSP_BF16) return fail(TSP_ERR_INVALID_ARG, "unknown dtype %d", s->dtype);
  return TSP_OK;
}

// K/V heads of the shape (Hkv = 0 stands for H).
int32_t kv_heads(const tsp_shape *s) { return s->Hkv ? s->Hkv : s->H; }

tsp_status check_attn_shape(const tsp_shape *s) {
  tsp_status st = check_axis(s);
  if (st) return st;
  if (s->H < 1) return fail(TSP_ERR_INVALID_ARG, "H=%d must be positive", s->H);
  if (s->Hkv < 0 || kv_heads(s) > s->H || s->H % kv_heads(s) != 0)
    return fail(TSP_ERR_INVALID_ARG, "Hkv=%d must divide H=%d (0 for Hkv = H)", s->Hkv, s->H);
  if (s->Dh != 64 && s->Dh != 128) return fail(TSP_ERR_UNSUPPORTED, "Dh=%d: only 64 and 128 are supported", s->Dh);
  if ((int64_t)s->H * s->Dh > (1 << 20)) return fail(TSP_ERR_INVALID_ARG, "H*Dh too large");
  if (!isfinite(s->scale) || s->scale < 0.f) return fail(TSP_ERR_INVALID_ARG, "scale must be finite and >= 0");
  return TSP_OK;
}

tsp_status check_mlp_shape(const tsp_shape *s) {
  tsp_status st = check_axis(s);
  if (st) return st;
  if (s->h < 64 || s->h % 64 != 0) return fail(TSP_ERR_UNSUPPORTED, "h=%d must be a positive multiple of 64", s->h);
  if (s->F < 1 || s->F % s->D != 0) return fail(TSP_ERR_INVALID_ARG, "F=%d must be a positive multiple of D=%d", s->F, s->D);
  if ((s->F / s->D) % 64 != 0) return fail(TSP_ERR_UNSUPPORTED, "F/D=%d must be a multiple of 64", s->F / s->D);
  if (s->mlp != TSP_MLP_GELU && s->mlp != TSP_MLP_SWIGLU) return fail(TSP_ERR_INVALID_ARG, "unknown mlp kind %d", s->mlp);
  if (s->mlp == TSP_MLP_SWIGLU && (int64_t)(2 * (s->F / s->D) + 256) * s->h * 2 >= ((int64_t)1 << 31))
    return fail(TSP_ERR_UNSUPPORTED, "gated MLP shard of %d x %d rows is too large", 2 * (s->F / s->D), s->h);
  return TSP_OK;
}

tsp_status check_layer_shape(const tsp_shape *s) {
  tsp_status st = check_attn_shape(s);
  if (st) return st;
  st = check_mlp_shape(s);
  if (st) return st;
  if (s->H % s->D != 0) return fail(TSP_ERR_INVALID_ARG, "H=%d must be a multiple of D=%d", s->H, s->D);
  if (kv_heads(s) % s->D != 0)
    return fail(TSP_ERR_INVALID_ARG, "Hkv=%d must be a multiple of D=%d", kv_heads(s), s->D);
  if (s->h != s->H * s->Dh) return fail(TSP_ERR_INVALID_ARG, "h=%d != H*Dh=%d", s->h, s->H * s->Dh);
  if (!isfinite(s->eps) || s->eps < 0.f) return fail(TSP_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!isfinite(s->rope_base) || s->rope_base < 0.f)
    return fail(TSP_ERR_INVALID_ARG, "rope_base must be finite and >= 0");
  if (s->rope_base > 0.f && s->dtype == TSP_BF16 &&
      ((s->h / s->D) % 128 != 0 || (kv_heads(s) / s->D * s->Dh) % 128 != 0))
    return fail(TSP_ERR_UNSUPPORTED, "rotary embedding in bf16 needs h/D=%d and Hkv*Dh/D=%d to be multiples of 128",
                s->h / s->D, kv_heads(s) / s->D * s->Dh);
  return TSP_OK;
}

// Rows of rank r recomputed in fp32 by the layer (bf16 rank 0 only): the
// positions below min(kLeadRows, S/(2D)), local rows 0.. of chunk 0.
int32_t lead_rows(const tsp_shape *s) {
  if (s->dtype != TSP_BF16 || s->r != 0) return 0;
  return (int32_t)std::min<int64_t>(tsp::kLeadRows, s->S / (2 * s->D));
}

struct LayerWs {
  size_t q, x2, hid;
  size_t rope;  // rotary table [N][Dh/2] (cos, sin) fp32, when rope_base > 0
  // leading rows: fp32 [m][h] normed input, q, k, v, attention output, h1,
  // normed h1; [m][F] hidden layer; partial sums of the products
  size_t la, lq, lk, lv, lo, lh1, lmm, lhid, lpart;
  size_t total;
};

LayerWs layer_ws(const tsp_shape *s) {
  const size_t e = elem_bytes(s->dtype);
  const size_t N = (size_t)(s->S / s->D);
  LayerWs w;
  w.q = 0;
  w.x2 = align256(N * s->h * e);
  w.hid = w.x2 + align256(N * s->h * e);
  size_t at = w.hid + align256(N * (size_t)s->F * e);
  w.rope = at;
  if (s->rope_base > 0.f) at += align256(N * (size_t)(s->Dh / 2) * 8);
  const size_t m = (size_t)lead_rows(s);
  const size_t mh = m ? align256(m * s->h * 4) : 0;
  w.la = at;
  w.lq = w.la + mh;
  w.lk = w.lq + mh;
  w.lv = w.lk + mh;
  w.lo = w.lv + mh;
  w.lh1 = w.lo + mh;
  w.lmm = w.lh1 + mh;
  w.lhid = w.lmm + mh;
  w.lpart = w.lhid + (m ? align256(m * (size_t)s->F * 4) : 0);
  w.total = w.lpart + (m ? align256(tsp::lead_part_bytes((int32_t)m, s->h, s->F, s->D, s->mlp == TSP_MLP_SWIGLU)) : 0);
  return w;
}

// GELU(x W1_j^T) of every ring step, [N][F] in ring-step column order.
size_t mlp_ws(const tsp_shape *s) {
  return align256((size_t)(s->S / s->D) * (size_t)s->F * elem_bytes(s->dtype));
}

// MLP backward scratch: the weights rearranged for the products (W1 stacked
// in ring order [F][h], its transpose [h][F], W2 transposed [F][h]), x^T and
// dy^T [h][N], Z^T (later dZ^T) and GELU(Z)^T [F][N]; the last also holds dZ
// [N][F] once GELU(Z)^T has been used.
struct MlpBwdWs {
  size_t w1cat, w1t, w2t, xt, dyt, zt, ht, total;
};

MlpBwdWs mlp_bwd_ws(const tsp_shape *s) {
  const size_t e = elem_bytes(s->dtype), N = (size_t)(s->S / s->D), h = (size_t)s->h, F = (size_t)s->F;
  MlpBwdWs w;
  w.w1cat = 0;
  w.w1t = w.w1cat + align256(F * h * e);
  w.w2t = w.w1t + align256(F * h * e);
  w.xt = w.w2t + align256(F * h * e);
  w.dyt = w.xt + align256(h * N * e);
  w.zt = w.dyt + align256(h * N * e);
  w.ht = w.zt + align256(F * N * e);
  w.total = w.ht + align256(F * N * e);
  return w;
}

// Attention backward scratch: log-sum-exp and Delta (sum of P dP) of every (head, row), fp32.
size_t attn_bwd_ws(const tsp_shape *s) { return 2 * align256((size_t)s->H * (size_t)(s->S / s->D) * 4); }

tsp_status check_mlp_bwd_shape(const tsp_shape *s) {
  tsp_status st = check_mlp_shape(s);
  if (st) return st;
  if (s->mlp != TSP_MLP_GELU) return fail(TSP_ERR_UNSUPPORTED, "the MLP backward covers the GELU MLP only");
  if ((s->S / s->D) % 64 != 0) return fail(TSP_ERR_UNSUPPORTED, "S/D=%lld must be a multiple of 64", (long long)(s->S / s->D));
  if ((int64_t)s->F * s->h >= (int64_t(1) << 31) / 2)
    return fail(TSP_ERR_UNSUPPORTED, "F*h=%lld is too large", (long long)s->F * s->h);
  // The layout passes put 64 rows of a matrix in one grid row (at most 65535
  // grid rows), and the products over K = tokens address 256 rows of N
  // tokens with 32-bit byte offsets: N, F and h are bounded here, before
  // anything is enqueued.
  const int64_t N = s->S / s->D, kMaxRows = int64_t(65535) * 64;
  if (N > kMaxRows || 256 * N * 2 >= (int64_t(1) << 31))
    return fail(TSP_ERR_UNSUPPORTED, "S/D=%lld is too large for the MLP backward", (long long)N);
  if (s->F > kMaxRows || s->h > kMaxRows)
    return fail(TSP_ERR_UNSUPPORTED, "F=%d or h=%d is too large for the MLP backward", s->F, s->h);
  return TSP_OK;
}

// Layer backward scratch: dh1 and dq (fp32) carried from TSP_BWD_ATTN to
// TSP_BWD_QKV, then one region that each phase lays out for itself.
//  ATTN: xn, Q, o (fp32) and o in dtype (panel), o^T, h1 (fp32), hn, dy in
//  dtype, dhn (fp32), dh1 in dtype (panel) and dh1^T (panel), W_O^T, do,
//  the forward's log-sum-exp, the attention backward's statistics, the gain
//  gradient partials and the MLP backward's own scratch.
//  QKV: xn, xn^T, [dq|dk|dv] (panel) and its transpose (panel), W_QKV^T,
//  dxn (fp32), the gain gradient partials.
struct LayerBwdWs {
  size_t dh1, dq;
  size_t xn, q, o, olo, ot, h1, hn, dylo, dhn, dh1lo, dh1t, wot, dout, lse, stat, part, mlp, mlp_bytes;
  size_t xr, xnt, dqkv, dqkvt, wqkvt, dxn, part2;
  size_t total;
};

LayerBwdWs layer_bwd_ws(const tsp_shape *s) {
  const size_t e = elem_bytes(s->dtype), N = (size_t)(s->S / s->D), h = (size_t)s->h;
  const size_t K3 = h + 2 * (size_t)kv_heads(s) * s->Dh;
  const size_t nh = align256(N * h * e), nh4 = align256(N * h * 4), part = align256(tsp::rmsnorm_bwd_part_bytes((int32_t)N, s->h));
  LayerBwdWs w;
  w.dh1 = 0;
  w.dq = nh4;
  const size_t region = 2 * nh4;
  size_t at = region;
  auto take = [&](size_t bytes) {
    const size_t o = at;
    at += bytes;
    return o;
  };
  w.xn = take(nh);
  w.q = take(nh);
  w.o = take(nh4);
  w.olo = take(nh);
  w.ot = take(nh);
  w.h1 = take(nh4);
  w.hn = take(nh);
  w.dylo = take(nh);
  w.dhn = take(nh4);
  w.dh1lo = take(nh);
  w.dh1t = take(nh);
  w.wot = take(align256(h * h * e));
  w.dout = take(nh);
  w.lse = take(align256((size_t)s->H * N * 4));
  w.stat = take(attn_bwd_ws(s));
  w.part = take(part);
  w.mlp_bytes = mlp_bwd_ws(s).total;
  w.mlp = take(w.mlp_bytes);
  const size_t attn_end = at;
  at = region;
  w.xr = take(nh);
  w.xnt = take(nh);
  w.dqkv = take(align256(N * K3 * e));
  w.dqkvt = take(align256(N * K3 * e));
  w.wqkvt = take(align256(h * K3 * e));
  w.dxn = take(nh4);
  w.part2 = take(part);
  w.total = std::max(attn_end, at);
  return w;
}

tsp_status check_layer_bwd_shape(const tsp_shape *s) {
  tsp_status st = check_layer_shape(s);
  if (st) return st;
  if ((st = check_mlp_bwd_shape(s))) return st;
  if (s->rope_base != 0.f) return fail(TSP_ERR_UNSUPPORTED, "the layer backward covers the layer without rotation");
  if (s->h > 8192) return fail(TSP_ERR_UNSUPPORTED, "h=%d: the RMSNorm backward takes h <= 8192", s->h);
  return TSP_OK;
}

tsp_status hip_fail(hipError_t e, const char *what) {
  return fail(TSP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

tsp::PtrList to_list(const void *const *p, int D) {
  tsp::PtrList l;
  memset(&l, 0, sizeof l);
  for (int j = 0; j < D; ++j) l.p[j] = p[j];
  return l;
}

// Shards in MLP ring order: entry t is the shard that reaches rank r at ring
// step t, j = (r - t) mod D (it arrives from rank r-1).
tsp::PtrList ring_list(const void *const *p, int D, int r) {
  tsp::PtrList l;
  memset(&l, 0, sizeof l);
  for (int t = 0; t < D; ++t) l.p[t] = p[((r - t) % D + D) % D];
  return l;
}

// ---------------------------------------------------------------- profiling
struct ProfRec {
  hipEvent_t a, b;
};
struct Prof {
  bool on = false;
  std::vector<ProfRec> open[TSP_K_COUNT];
  std::vector<hipEvent_t> pool;
  double ms[TSP_K_COUNT] = {};
  int64_t n[TSP_K_COUNT] = {};
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void drain(int k) {
    for (ProfRec &r : open[k]) {
      if (r.a && r.b && hipEventSynchronize(r.b) == hipSuccess) {
        float t = 0.f;
        if (hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
          ms[k] += t;
          n[k] += 1;
        }
      }
      if (r.a) pool.push_back(r.a);
      if (r.b) pool.push_back(r.b);
    }
    open[k].clear();
  }
};
Prof g_prof;

}  // namespace

namespace tsp {
void prof_begin(int k, hipStream_t s) {
  if (!g_prof.on) return;
  ProfRec r{g_prof.get(), nullptr};
  if (r.a && hipEventRecord(r.a, s) != hipSuccess) {  // not timed, the launch still runs
    g_prof.pool.push_back(r.a);
    r.a = nullptr;
  }
  g_prof.open[k].push_back(r);
}
void prof_end(int k, hipStream_t s) {
  if (!g_prof.on || g_prof.open[k].empty()) return;
  ProfRec &r = g_prof.open[k].back();
  r.b = g_prof.get();
  if (r.b && hipEventRecord(r.b, s) != hipSuccess) {
    g_prof.pool.push_back(r.b);
    r.b = nullptr;
  }
}
}  // namespace tsp

#define TSP_LAUNCH(kclass, call, what)                \
  do {                                                \
    tsp::prof_begin(kclass, stream);                  \
    hipError_t e_ = (call);                           \
    tsp::prof_end(kclass, stream);                    \
    if (e_ != hipSuccess) return hip_fail(e_, what);  \
  } while (0)

extern "C" {

const char *tsp_status_string(int status) {
  switch (status) {
    case TSP_OK: return "ok";
    case TSP_ERR_INVALID_ARG: return "invalid argument";
    case TSP_ERR_UNSUPPORTED: return "unsupported shape";
    case TSP_ERR_WORKSPACE: return "workspace too small";
    case TSP_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *tsp_last_error(void) { return g_err.c_str(); }

int tsp_abi_version(void) { return 3; }

tsp_status tsp_workspace_size(const tsp_shape *s, int which, size_t *bytes) {
  if (!bytes) return fail(TSP_ERR_INVALID_ARG, "bytes is NULL");
  tsp_status st;
  if (which == TSP_WS_MLP) {
    if ((st = check_mlp_shape(s))) return st;
    *bytes = mlp_ws(s);
  } else if (which == TSP_WS_LAYER) {
    if ((st = check_layer_shape(s))) return st;
    *bytes = layer_ws(s).total;
  } else if (which == TSP_WS_MLP_BWD) {
    if ((st = check_mlp_bwd_shape(s))) return st;
    *bytes = mlp_bwd_ws(s).total;
  } else if (which == TSP_WS_ATTN_BWD) {
    if ((st = check_attn_shape(s))) return st;
    *bytes = attn_bwd_ws(s);
  } else if (which == TSP_WS_LAYER_BWD) {
    if ((st = check_layer_bwd_shape(s))) return st;
    *bytes = layer_bwd_ws(s).total;
  } else {
    return fail(TSP_ERR_INVALID_ARG, "unknown workspace kind %d", which);
  }
  return ok();
}

tsp_status tsp_zigzag_index_host(int64_t S, int32_t D, int32_t r, int32_t *pos) {
  tsp_shape s{};
  s.S = S;
  s.D = D;
  s.r = r;
  s.dtype = TSP_F32;
  tsp_status st = check_axis(&s);
  if (st) return st;
  if (!pos) return fail(TSP_ERR_INVALID_ARG, "pos is NULL");
  const tsp::ZigzagMap zz = tsp::make_zigzag(S, D, r);
  const int32_t n = (int32_t)(S / D);
  for (int32_t t = 0; t < n; ++t) pos[t] = zz.pos(t);
  return ok();
}

tsp_status tsp_zigzag_index(int64_t S, int32_t D, int32_t r, int32_t *pos, void *stream_) {
  tsp_shape s{};
  s.S = S;
  s.D = D;
  s.r = r;
  s.dtype = TSP_F32;
  tsp_status st = check_axis(&s);
  if (st) return st;
  if ((st = check_ptr(pos, "pos"))) return st;
  hipStream_t stream = (hipStream_t)stream_;
  TSP_LAUNCH(TSP_K_ZIGZAG, tsp::launch_zigzag_index(tsp::make_zigzag(S, D, r), (int32_t)(S / D), pos, stream),
             "zigzag index");
  return ok();
}

tsp_status tsp_zigzag_attn(const tsp_shape *s, const void *q, const void *k, const void *v, void *o,
                           int32_t o_dtype, void *stream_) {
  return tsp_zigzag_attn_ex(s, q, k, v, o, o_dtype, 0u, stream_);
}

tsp_status tsp_zigzag_attn_ex(const tsp_shape *s, const void *q, const void *k, const void *v, void *o,
                              int32_t o_dtype, uint32_t flags, void *stream_) {
  tsp_status st = check_attn_shape(s);
  if (st) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(o, "o")))
    return st;
  if (o_dtype != TSP_F32 && o_dtype != TSP_BF16) return fail(TSP_ERR_INVALID_ARG, "unknown o_dtype %d", o_dtype);
  if (s->dtype == TSP_F32 && o_dtype != TSP_F32) return fail(TSP_ERR_INVALID_ARG, "fp32 inputs need an fp32 output");
  if (flags & ~(uint32_t)TSP_ATTN_Q_LOG2_SCALED) return fail(TSP_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const bool q_log2 = (flags & TSP_ATTN_Q_LOG2_SCALED) != 0;
  if (q_log2 && (s->dtype != TSP_BF16 || o_dtype != TSP_BF16))
    return fail(TSP_ERR_UNSUPPORTED, "TSP_ATTN_Q_LOG2_SCALED needs bf16 q and o");
  const size_t e = elem_bytes(s->dtype), row = (size_t)s->H * s->Dh, kvrow = (size_t)kv_heads(s) * s->Dh;
  const size_t N = (size_t)(s->S / s->D);
  const Range ro{o, N * row * elem_bytes(o_dtype), "o"};
  const Range ins[] = {
      {q, N * row * e, "q"}, {k, (size_t)s->S * kvrow * e, "k"}, {v, (size_t)s->S * kvrow * e, "v"}};
  for (const Range &r : ins)
    if (overlap(ro, r)) return fail(TSP_ERR_INVALID_ARG, "o overlaps %s", r.name);
  hipStream_t stream = (hipStream_t)stream_;
  TSP_LAUNCH(TSP_K_ATTN,
             tsp::launch_attention(s->dtype, q, k, v, o, o_dtype, false, s->S, (int32_t)N, s->H, kv_heads(s), s->Dh,
                                   s->scale, tsp::make_zigzag(s->S, s->D, s->r), q_log2, stream),
             "attention");
  return ok();
}

static tsp_status mlp_ring(const tsp_shape *s, const void *x, const void *const *w1, const void *const *w2,
                           const float *residual, float *y, void *z, void *ws, size_t ws_bytes, void *stream_) {
  tsp_status st = check_mlp_shape(s);
  if (st) return st;
  if ((st = check_ptr(x, "x")) || (st = check_ptr(y, "y")) || (st = check_ptr(ws, "ws"))) return st;
  if (residual && !aligned16(residual)) return fail(TSP_ERR_INVALID_ARG, "residual is not 16-byte aligned");
  if (z) {
    if ((st = check_ptr(z, "z"))) return st;
    if (s->dtype != TSP_BF16 || s->mlp != TSP_MLP_GELU)
      return fail(TSP_ERR_UNSUPPORTED, "the pre-activation output covers the bf16 GELU MLP only");
  }
  if ((st = check_ptr_list(w1, s->D, "w1")) || (st = check_ptr_list(w2, s->D, "w2"))) return st;
  const size_t need = mlp_ws(s);
  if (ws_bytes < need) return fail(TSP_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, need);
  const int32_t N = (int32_t)(s->S / s->D), h = s->h, fd = s->F / s->D;
  const Range ry{y, (size_t)N * h * 4, "y"}, rx{x, (size_t)N * h * elem_bytes(s->dtype), "x"}, rw{ws, need, "ws"};
  if (overlap(ry, rx) || overlap(ry, rw) || overlap(rx, rw))
    return fail(TSP_ERR_INVALID_ARG, "x, y and ws must not overlap");
  if (residual && residual != y && overlap(Range{residual, (size_t)N * h * 4, "residual"}, ry))
    return fail(TSP_ERR_INVALID_ARG, "residual overlaps y without being equal to it");
  const Range rz{z, (size_t)N * s->F * 2, "z"};
  if (overlap(rz, rx) || overlap(rz, ry) || overlap(rz, rw) ||
      (residual && overlap(rz, Range{residual, (size_t)N * h * 4, "residual"})))
    return fail(TSP_ERR_INVALID_ARG, "z overlaps x, y, residual or ws");
  hipStream_t stream = (hipStream_t)stream_;
  // every ring step's GELU(x W1_j^T) side by side (bf16: in 64-column
  // panels), then one reduction over them and the W2 shards in ring order
  const bool pnl = s->dtype == TSP_BF16;
  TSP_LAUNCH(TSP_K_MLP_UP,
             tsp::launch_mlp_up(s->dtype, x, false, N, h, ring_list(w1, s->D, s->r), s->D, fd, s->mlp == TSP_MLP_SWIGLU,
                                ws, pnl, stream, z),
             "MLP up");
  TSP_LAUNCH(TSP_K_MLP_DOWN,
             tsp::launch_mlp_down(s->dtype, ws, pnl, N, ring_list(w2, s->D, s->r), s->D, fd, h, residual, y, stream),
             "MLP down");
  return ok();
}

tsp_status tsp_zigzag_attn_lse(const tsp_shape *s, const void *q, const void *k, const void *v, float *o, float *lse,
                               void *stream_) {
  tsp_status st = check_attn_shape(s);
  if (st) return st;
  if (s->dtype != TSP_BF16) return fail(TSP_ERR_UNSUPPORTED, "tsp_zigzag_attn_lse takes bf16 inputs");
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(o, "o")) ||
      (st = check_ptr(lse, "lse")))
    return st;
  const size_t row = (size_t)s->H * s->Dh, kvrow = (size_t)kv_heads(s) * s->Dh, N = (size_t)(s->S / s->D);
  const Range outs[] = {{o, N * row * 4, "o"}, {lse, N * s->H * 4, "lse"}};
  const Range ins[] = {{q, N * row * 2, "q"}, {k, (size_t)s->S * kvrow * 2, "k"}, {v, (size_t)s->S * kvrow * 2, "v"}};
  for (const Range &ro : outs)
    for (const Range &ri : ins)
      if (overlap(ro, ri)) return fail(TSP_ERR_INVALID_ARG, "%s overlaps %s", ro.name, ri.name);
  if (overlap(outs[0], outs[1])) return fail(TSP_ERR_INVALID_ARG, "o overlaps lse");
  hipStream_t stream = (hipStream_t)stream_;
  TSP_LAUNCH(TSP_K_ATTN,
             tsp::launch_attention(s->dtype, q, k, v, o, TSP_F32, false, s->S, (int32_t)N, s->H, kv_heads(s), s->Dh,
                                   s->scale, tsp::make_zigzag(s->S, s->D, s->r), false, stream, lse),
             "attention");
  return ok();
}

// ws == nullptr with static_ws: the scratch is the library's static device
// array (tsp_zigzag_attn_bwd_noalloc), looked up after every argument check.
static tsp_status attn_bwd(const tsp_shape *s, const void *q, const void *k, const void *v, const float *o, const float *lse,
                    const void *dout, float *dq, float *dk, float *dv, void *ws, size_t ws_bytes, void *stream_,
                    bool static_ws = false, uint32_t flags = 0) {
  tsp_status st = check_attn_shape(s);
  if (st) return st;
  if (flags & ~(uint32_t)TSP_ATTN_BWD_PLAIN_PDS) return fail(TSP_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const bool plain = (flags & TSP_ATTN_BWD_PLAIN_PDS) != 0;
  if (plain && s->dtype != TSP_BF16) return fail(TSP_ERR_UNSUPPORTED, "TSP_ATTN_BWD_PLAIN_PDS takes bf16 inputs");
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(dout, "dout")) ||
      (st = check_ptr(dq, "dq")) || (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")) ||
      (!static_ws && (st = check_ptr(ws, "ws"))))
    return st;
  const bool given = o != nullptr || lse != nullptr;
  if (given) {
    if ((st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse"))) return st;
    if (s->dtype != TSP_BF16) return fail(TSP_ERR_UNSUPPORTED, "the forward's statistics are taken with bf16 inputs");
  }
  const size_t need = attn_bwd_ws(s);
  if (static_ws && need > tsp::kNoallocScratchBytes)
    return fail(TSP_ERR_UNSUPPORTED,
                "H*S/D=%lld rows of statistics need %zu bytes of scratch, more than the static %zu (H*S/D <= %zu)",
                (long long)s->H * (s->S / s->D), need, tsp::kNoallocScratchBytes, tsp::kNoallocScratchBytes / 8);
  if (!static_ws && ws_bytes < need) return fail(TSP_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, need);
  const int64_t N = s->S / s->D;
  const size_t e = elem_bytes(s->dtype);
  const size_t qb = (size_t)N * s->H * s->Dh, kb = (size_t)s->S * kv_heads(s) * s->Dh;
  const Range ins[] = {{q, qb * e, "q"},       {k, kb * e, "k"},   {v, kb * e, "v"},
                       {dout, qb * e, "dout"}, {o, qb * 4, "o"},   {lse, (size_t)N * s->H * 4, "lse"}};
  const Range outs[] = {{dq, qb * 4, "dq"}, {dk, kb * 4, "dk"}, {dv, kb * 4, "dv"},
                        {static_ws ? nullptr : ws, need, "ws"}};
  for (const Range &ro : outs) {
    for (const Range &ri : ins)
      if (overlap(ro, ri)) return fail(TSP_ERR_INVALID_ARG, "%s overlaps %s", ro.name, ri.name);
    for (const Range &r2 : outs)
      if (&r2 != &ro && overlap(ro, r2)) return fail(TSP_ERR_INVALID_ARG, "%s overlaps %s", ro.name, r2.name);
  }
  hipStream_t stream = (hipStream_t)stream_;
  if (static_ws) {
    const hipError_t e_ = tsp::noalloc_scratch(stream, &ws);
    if (e_ == hipErrorInvalidDevice)
      return fail(TSP_ERR_INVALID_ARG, "the stream's device is not the current device (or above 64)");
    if (e_ != hipSuccess) return hip_fail(e_, "static scratch lookup");
  }
  float *lse_ws = (float *)ws, *delta = (float *)((unsigned char *)ws + need / 2);
  TSP_LAUNCH(TSP_K_ATTN_BWD,
             tsp::launch_attention_bwd(s->dtype, q, k, v, dout, dq, dk, dv, lse_ws, delta, s->S, (int32_t)N, s->H,
                                       kv_heads(s), s->Dh, s->scale, tsp::make_zigzag(s->S, s->D, s->r), stream, o,
                                       lse, !plain),
             "attention backward");
  return ok();
}

tsp_status tsp_zigzag_attn_bwd(const tsp_shape *s, const void *q, const void *k, const void *v, const void *dout,
                               float *dq, float *dk, float *dv, void *ws, size_t ws_bytes, void *stream) {
  return attn_bwd(s, q, k, v, nullptr, nullptr, dout, dq, dk, dv, ws, ws_bytes, stream);
}

tsp_status tsp_zigzag_attn_bwd_noalloc(const tsp_shape *s, const void *q, const void *k, const void *v, const void *dout,
                                       float *dq, float *dk, float *dv, void *stream) {
  return attn_bwd(s, q, k, v, nullptr, nullptr, dout, dq, dk, dv, nullptr, 0, stream, true);
}

tsp_status tsp_zigzag_attn_bwd_ex(const tsp_shape *s, const void *q, const void *k, const void *v, const float *o,
                                  const float *lse, const void *dout, float *dq, float *dk, float *dv, uint32_t flags,
                                  void *ws, size_t ws_bytes, void *stream) {
  if ((o == nullptr) != (lse == nullptr)) return fail(TSP_ERR_INVALID_ARG, "%s is NULL", o ? "lse" : "o");
  return attn_bwd(s, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, stream, false, flags);
}

tsp_status tsp_zigzag_attn_bwd_lse(const tsp_shape *s, const void *q, const void *k, const void *v, const float *o,
                                   const float *lse, const void *dout, float *dq, float *dk, float *dv, void *ws,
                                   size_t ws_bytes, void *stream) {
  if (!o || !lse) return fail(TSP_ERR_INVALID_ARG, "%s is NULL", o ? "lse" : "o");
  return attn_bwd(s, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, stream);
}

static tsp_status mlp_ring_bwd(const tsp_shape *s, const void *x, const void *zin, const void *const *w1,
                               const void *const *w2, const void *dy, const float *dx_residual, float *dx,
                               float *const *dw1, float *const *dw2, void *ws, size_t ws_bytes, void *stream_) {
  tsp_status st = check_mlp_bwd_shape(s);
  if (st) return st;
  if ((st = check_ptr(x, "x")) || (st = check_ptr(dy, "dy")) || (st = check_ptr(dx, "dx")) ||
      (st = check_ptr(ws, "ws")))
    return st;
  if (dx_residual && !aligned16(dx_residual)) return fail(TSP_ERR_INVALID_ARG, "dx_residual is not 16-byte aligned");
  if (zin) {
    if ((st = check_ptr(zin, "z"))) return st;
    if (s->dtype != TSP_BF16) return fail(TSP_ERR_UNSUPPORTED, "a given pre-activation needs bf16");
  }
  if ((st = check_ptr_list(w1, s->D, "w1")) || (st = check_ptr_list(w2, s->D, "w2")) ||
      (st = check_ptr_list((const void *const *)dw1, s->D, "dw1")) ||
      (st = check_ptr_list((const void *const *)dw2, s->D, "dw2")))
    return st;
  const MlpBwdWs L = mlp_bwd_ws(s);
  if (ws_bytes < L.total) return fail(TSP_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, L.total);
  const int32_t N = (int32_t)(s->S / s->D), h = s->h, F = s->F, D = s->D, fd = F / D;
  const size_t e = elem_bytes(s->dtype);
  const Range rdx{dx, (size_t)N * h * 4, "dx"}, rx{x, (size_t)N * h * e, "x"}, rdy{dy, (size_t)N * h * e, "dy"},
      rw{ws, L.total, "ws"};
  if (overlap(rdx, rx) || overlap(rdx, rdy) || overlap(rdx, rw) || overlap(rx, rw) || overlap(rdy, rw))
    return fail(TSP_ERR_INVALID_ARG, "x, dy, dx and ws must not overlap");
  const Range rz{zin, (size_t)N * F * 2, "z"};
  if (overlap(rz, rdx) || overlap(rz, rw)) return fail(TSP_ERR_INVALID_ARG, "z overlaps dx or ws");
  if (dx_residual && dx_residual != dx && overlap(Range{dx_residual, (size_t)N * h * 4, "dx_residual"}, rdx))
    return fail(TSP_ERR_INVALID_ARG, "dx_residual overlaps dx without being equal to it");
  for (int j = 0; j < D; ++j) {
    const Range r1{dw1[j], (size_t)fd * h * 4, "dw1"}, r2{dw2[j], (size_t)h * fd * 4, "dw2"};
    if (overlap(r1, rw) || overlap(r2, rw) || overlap(r1, rdx) || overlap(r2, rdx))
      return fail(TSP_ERR_INVALID_ARG, "dw1[%d]/dw2[%d] overlap dx or ws", j, j);
  }
  hipStream_t stream = (hipStream_t)stream_;
  unsigned char *base = (unsigned char *)ws;
  void *w1cat = base + L.w1cat, *w1t = base + L.w1t, *w2t = base + L.w2t, *xt = base + L.xt, *dyt = base + L.dyt,
       *zt = base + L.zt, *ht = base + L.ht;
  const bool bf = s->dtype == TSP_BF16;
  const tsp::PtrList r1 = ring_list(w1, D, s->r), r2 = ring_list(w2, D, s->r);
  // weights in ring-step order: W1 rows stacked (for the recomputation of Z),
  // W1^T and W2^T
  for (int t = 0; t < D && !zin; ++t) {
    hipError_t err = hipMemcpyAsync(base + L.w1cat + (size_t)t * fd * h * e, r1.p[t], (size_t)fd * h * e,
                                    hipMemcpyDeviceToDevice, stream);
    if (err != hipSuccess) return hip_fail(err, "W1 copy");
  }
  TSP_LAUNCH(TSP_K_TRANSPOSE, tsp::launch_transpose(s->dtype, r1, D, h, 0, fd, h, w1t, F, 0, fd, stream), "W1 transpose");
  TSP_LAUNCH(TSP_K_TRANSPOSE,
             tsp::launch_transpose(s->dtype, r2, D, fd, 0, h, fd, w2t, h, 0, (int64_t)fd * h, stream), "W2 transpose");
  // activations with the token axis innermost (K of the weight gradients)
  tsp::PtrList lx{}, ldy{};
  lx.p[0] = x;
  ldy.p[0] = dy;
  TSP_LAUNCH(TSP_K_TRANSPOSE, tsp::launch_transpose(s->dtype, lx, 1, h, 0, N, h, xt, N, 0, 0, stream), "x transpose");
  TSP_LAUNCH(TSP_K_TRANSPOSE,
             tsp::launch_transpose(s->dtype, ldy, 1, h, 0, N, h, dyt, N, bf ? (int64_t)h * 64 : 0, 0, stream),
             "dy transpose");
  // Z^T and GELU(Z)^T (recomputed, or from the given Z), then
  // dZ^T = (W2^T dy^T) * GELU'(Z^T) in place
  if (zin)
    TSP_LAUNCH(TSP_K_TRANSPOSE, tsp::launch_transpose_gelu(zin, N, F, zt, ht, stream), "Z transpose");
  else
    TSP_LAUNCH(TSP_K_BWD_GEMM, tsp::launch_mlp_bwd_recompute(s->dtype, w1cat, F, h, x, N, zt, bf, ht, stream),
               "MLP backward Z");
  TSP_LAUNCH(TSP_K_BWD_GEMM, tsp::launch_mlp_bwd_dz(s->dtype, w2t, F, h, dy, N, zt, bf, stream), "MLP backward dZ");
  // weight gradients of every ring step's shard: dW1 = dZ^T x, dW2 = dy^T GELU(Z)
  TSP_LAUNCH(TSP_K_BWD_GEMM,
             tsp::launch_wgrad(s->dtype, zt, bf, F, xt, h, N, ring_list((const void *const *)dw1, D, s->r), fd, true,
                               stream),
             "MLP backward dW1");
  TSP_LAUNCH(TSP_K_BWD_GEMM,
             tsp::launch_wgrad(s->dtype, dyt, bf, h, ht, F, N, ring_list((const void *const *)dw2, D, s->r), fd, false,
                               stream),
             "MLP backward dW2");
  // dZ [N][F] over the GELU(Z)^T buffer, then dx = dZ W1 reduced in ring order
  tsp::PtrList lz{};
  lz.p[0] = zt;
  TSP_LAUNCH(TSP_K_TRANSPOSE,
             tsp::launch_transpose(s->dtype, lz, 1, N, bf ? (int64_t)F * 64 : 0, F, N, ht, F, bf ? (int64_t)N * 64 : 0,
                                   0, stream),
             "dZ transpose");
  TSP_LAUNCH(TSP_K_BWD_GEMM, tsp::launch_mlp_bwd_dx(s->dtype, ht, bf, N, F, w1t, h, dx_residual, dx, stream),
             "MLP backward dx");
  return ok();
}

tsp_status tsp_mlp_ring(const tsp_shape *s, const void *x, const void *const *w1, const void *const *w2,
                        const float *residual, float *y, void *ws, size_t ws_bytes, void *stream) {
  return mlp_ring(s, x, w1, w2, residual, y, nullptr, ws, ws_bytes, stream);
}

tsp_status tsp_mlp_ring_z(const tsp_shape *s, const void *x, const void *const *w1, const void *const *w2,
                          const float *residual, float *y, void *z, void *ws, size_t ws_bytes, void *stream) {
  if (!z) return fail(TSP_ERR_INVALID_ARG, "z is NULL");
  return mlp_ring(s, x, w1, w2, residual, y, z, ws, ws_bytes, stream);
}

tsp_status tsp_mlp_ring_bwd(const tsp_shape *s, const void *x, const void *const *w1, const void *const *w2,
                            const void *dy, const float *dx_residual, float *dx, float *const *dw1, float *const *dw2,
                            void *ws, size_t ws_bytes, void *stream) {
  return mlp_ring_bwd(s, x, nullptr, w1, w2, dy, dx_residual, dx, dw1, dw2, ws, ws_bytes, stream);
}

tsp_status tsp_mlp_ring_bwd_z(const tsp_shape *s, const void *x, const void *z, const void *const *w1,
                              const void *const *w2, const void *dy, const float *dx_residual, float *dx,
                              float *const *dw1, float *const *dw2, void *ws, size_t ws_bytes, void *stream) {
  if (!z) return fail(TSP_ERR_INVALID_ARG, "z is NULL");
  return mlp_ring_bwd(s, x, z, w1, w2, dy, dx_residual, dx, dw1, dw2, ws, ws_bytes, stream);
}

// The layer forward; with o_save and lse_save (bf16), the attention also
// writes its fp32 output and the rows' natural log-sum-exp there for the
// backward, and the output projection reads O packed from o_save.
static tsp_status layer_fwd(const tsp_shape *s, const tsp_layer_weights *w, const float *x, void *k_full,
                            void *v_full, float *y, float *o_save, float *lse_save, void *z_save, unsigned phases,
                            void *ws_, size_t ws_bytes, void *stream_) {
  tsp_status st = check_layer_shape(s);
  if (st) return st;
  const bool save = o_save != nullptr || lse_save != nullptr;
  if (save && (!o_save || !lse_save)) return fail(TSP_ERR_INVALID_ARG, "o_save and lse_save must both be given");
  if (save && s->dtype != TSP_BF16) return fail(TSP_ERR_UNSUPPORTED, "saving the attention output needs bf16");
  if (save && ((st = check_ptr(o_save, "o_save")) || (st = check_ptr(lse_save, "lse_save")))) return st;
  if (z_save) {
    if (!save) return fail(TSP_ERR_INVALID_ARG, "z_save needs o_save and lse_save");
    if (s->mlp != TSP_MLP_GELU) return fail(TSP_ERR_UNSUPPORTED, "keeping the MLP pre-activation needs the GELU MLP");
    if ((st = check_ptr(z_save, "z_save"))) return st;
  }
  if (!w) return fail(TSP_ERR_INVALID_ARG, "weights is NULL");
  if (phases == 0 || (phases & ~3u)) return fail(TSP_ERR_INVALID_ARG, "phases=%u must be 1, 2 or 3", phases);
  if ((st = check_ptr(x, "x")) || (st = check_ptr(k_full, "k_full")) || (st = check_ptr(v_full, "v_full")) ||
      (st = check_ptr(y, "y")) || (st = check_ptr(ws_, "ws")) || (st = check_ptr(w->g_attn, "g_attn")) ||
      (st = check_ptr(w->g_mlp, "g_mlp")))
    return st;
  if ((st = check_ptr_list(w->wqkv, s->D, "wqkv")) || (st = check_ptr_list(w->wo, s->D, "wo")) ||
      (st = check_ptr_list(w->w1, s->D, "w1")) || (st = check_ptr_list(w->w2, s->D, "w2")))
    return st;
  const LayerWs L = layer_ws(s);
  if (ws_bytes < L.total) return fail(TSP_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, L.total);
  const int32_t N = (int32_t)(s->S / s->D), h = s->h, D = s->D, hd = h / D, fd = s->F / D;
  // K/V: Hkv heads, hk = Hkv*Dh/D columns per shard, rows of hkv = Hkv*Dh
  const int32_t Hkv = kv_heads(s), hkv = Hkv * s->Dh, hk = hkv / D;
  const bool gated = s->mlp == TSP_MLP_SWIGLU;
  const size_t e = elem_bytes(s->dtype);
  const Range rx{x, (size_t)N * h * 4, "x"}, ry{y, (size_t)N * h * 4, "y"}, rws{ws_, L.total, "ws"};
  const Range rk{k_full, (size_t)s->S * hkv * e, "k_full"}, rv{v_full, (size_t)s->S * hkv * e, "v_full"};
  const Range ro{o_save, save ? (size_t)N * h * 4 : 0, "o_save"};
  const Range rl{lse_save, save ? (size_t)s->H * N * 4 : 0, "lse_save"};
  const Range rz{z_save, z_save ? (size_t)N * s->F * 2 : 0, "z_save"};
  const Range all[] = {rx, ry, rws, rk, rv, ro, rl, rz};
  const int n_ranges = z_save ? 8 : save ? 7 : 5;
  for (int i = 0; i < n_ranges; ++i)
    for (int j = i + 1; j < n_ranges; ++j)
      if (overlap(all[i], all[j])) return fail(TSP_ERR_INVALID_ARG, "%s overlaps %s", all[i].name, all[j].name);

  unsigned char *ws = static_cast<unsigned char *>(ws_);
  // With bf16, every activation that a GEMM reads as its A operand (x2, O,
  // RMSNorm(h1), H) is kept in 64-column panels; Q stays [N][H][Dh].
  void *qbuf = ws + L.q;   // Q, later RMSNorm(h1)
  void *x2 = ws + L.x2;    // RMSNorm(x), later the attention output O
  void *hid = ws + L.hid;  // GELU(hn W1_j^T) of every ring step, side by side
  const tsp::ZigzagMap zz = tsp::make_zigzag(s->S, D, s->r);
  const bool pnl = s->dtype == TSP_BF16;
  // bf16: the QKV epilogue stores Q * scale * log2(e), so attention's scores
  // come out of the matrix cores in the log2 domain (one rounding of Q, as
  // without the factor)
  const float q_scale = pnl ? s->scale * 1.4426950408889634f : 1.0f;
  hipStream_t stream = (hipStream_t)stream_;

  // rotary table, written with the QKV of PHASE_KV and read again by the
  // leading rows in PHASE_REST (same ws)
  const bool rope = s->rope_base > 0.f;
  float2 *rtab = rope ? reinterpret_cast<float2 *>(ws + L.rope) : nullptr;
  if (phases & TSP_PHASE_KV) {
    TSP_LAUNCH(TSP_K_RMSNORM, tsp::launch_rmsnorm(x, w->g_attn, x2, N, h, s->eps, s->dtype, pnl, stream), "RMSNorm");
    if (rope)
      TSP_LAUNCH(TSP_K_QKV, tsp::launch_rope_table(zz, N, s->Dh, s->rope_base, rtab, stream), "rotary table");
    // bf16: Q and K are rotated in the QKV epilogue, before rounding; fp32:
    // in place afterwards
    TSP_LAUNCH(TSP_K_QKV,
               tsp::launch_qkv(s->dtype, x2, pnl, N, h, to_list(w->wqkv, D), D, hd, hk, qbuf, k_full, v_full, zz,
                               q_scale, pnl ? rtab : nullptr, s->Dh, stream),
               "QKV");
    if (rope && !pnl) {
      TSP_LAUNCH(TSP_K_QKV, tsp::launch_rope_rows((float *)qbuf, h, N, s->H, s->Dh, zz, false, rtab, stream),
                 "rotary embedding of Q");
      TSP_LAUNCH(TSP_K_QKV, tsp::launch_rope_rows((float *)k_full, hkv, N, Hkv, s->Dh, zz, true, rtab, stream),
                 "rotary embedding of K");
    }
  }
  if (phases & TSP_PHASE_REST) {
    if (save) {  // the same attention, fp32 O and the row statistics kept; O to bf16 panels
      TSP_LAUNCH(TSP_K_ATTN,
                 tsp::launch_attention(s->dtype, qbuf, k_full, v_full, o_save, TSP_F32, false, s->S, N, s->H, Hkv,
                                       s->Dh, s->scale, zz, true, stream, lse_save),
                 "attention");
      TSP_LAUNCH(TSP_K_ROWS_BWD, tsp::launch_pack_cols(s->dtype, o_save, nullptr, nullptr, N, 1, h, 0, x2, true, stream),
                 "o conversion");
    } else {
      TSP_LAUNCH(TSP_K_ATTN,
                 tsp::launch_attention(s->dtype, qbuf, k_full, v_full, x2, s->dtype, pnl, s->S, N, s->H, Hkv, s->Dh,
                                       s->scale, zz, pnl, stream),
                 "attention");
    }
    TSP_LAUNCH(TSP_K_OUTPROJ,
               tsp::launch_outproj(s->dtype, x2, pnl, N, h, to_list(w->wo, D), D, hd, x, y, stream),
               "output projection");
    TSP_LAUNCH(TSP_K_RMSNORM, tsp::launch_rmsnorm(y, w->g_mlp, qbuf, N, h, s->eps, s->dtype, pnl, stream),
               "RMSNorm");
    TSP_LAUNCH(TSP_K_MLP_UP,
               tsp::launch_mlp_up(s->dtype, qbuf, pnl, N, h, ring_list(w->w1, D, s->r), D, fd, gated, hid, pnl, stream,
                                  z_save),
               "MLP up");
    TSP_LAUNCH(TSP_K_MLP_DOWN,
               tsp::launch_mlp_down(s->dtype, hid, pnl, N, ring_list(w->w2, D, s->r), D, fd, h, y, y, stream),
               "MLP down");
    const int32_t m = lead_rows(s);
    if (m > 0) {
      // rank 0's first m rows again, fp32 throughout; they attend only to
      // each other (positions 0..m-1), so their K/V come from the same pass
      float *la = (float *)(ws + L.la), *lq = (float *)(ws + L.lq), *lk = (float *)(ws + L.lk);
      float *lv = (float *)(ws + L.lv), *lo = (float *)(ws + L.lo), *lh1 = (float *)(ws + L.lh1);
      float *lmm = (float *)(ws + L.lmm), *lhid = (float *)(ws + L.lhid), *lpart = (float *)(ws + L.lpart);
      TSP_LAUNCH(TSP_K_LEAD, tsp::launch_rmsnorm_f32(x, w->g_attn, s->dtype, la, m, h, s->eps, stream),
                 "leading rows: RMSNorm");
      TSP_LAUNCH(TSP_K_LEAD,
                 tsp::launch_lead_qkv(la, m, h, to_list(w->wqkv, D), D, hd, hk, lq, lk, lv, zz, lpart, stream),
                 "leading rows: QKV");
      if (rope) {  // rows 0..m-1 sit at positions 0..m-1, table rows 0..m-1
        TSP_LAUNCH(TSP_K_LEAD, tsp::launch_rope_rows(lq, h, m, s->H, s->Dh, zz, false, rtab, stream),
                   "leading rows: rotary embedding of Q");
        TSP_LAUNCH(TSP_K_LEAD, tsp::launch_rope_rows(lk, hkv, m, Hkv, s->Dh, zz, false, rtab, stream),
                   "leading rows: rotary embedding of K");
      }
      TSP_LAUNCH(TSP_K_LEAD,
                 tsp::launch_lead_attention(lq, lk, lv, lo, m, s->H, Hkv, s->Dh, s->scale, stream),
                 "leading rows: attention");
      TSP_LAUNCH(TSP_K_LEAD, tsp::launch_lead_outproj(lo, m, h, to_list(w->wo, D), D, hd, x, lh1, lpart, stream),
                 "leading rows: output projection");
      TSP_LAUNCH(TSP_K_LEAD, tsp::launch_rmsnorm_f32(lh1, w->g_mlp, s->dtype, lmm, m, h, s->eps, stream),
                 "leading rows: RMSNorm");
      TSP_LAUNCH(TSP_K_LEAD,
                 tsp::launch_lead_mlp_up(lmm, m, h, ring_list(w->w1, D, s->r), D, fd, gated, lhid, lpart, stream),
                 "leading rows: MLP up");
      TSP_LAUNCH(TSP_K_LEAD,
                 tsp::launch_lead_mlp_down(lhid, m, ring_list(w->w2, D, s->r), D, fd, h, lh1, y, lpart, stream),
                 "leading rows: MLP down");
    }
  }
  return ok();
}

tsp_status tsp_layer_fwd(const tsp_shape *s, const tsp_layer_weights *w, const float *x, void *k_full,
                         void *v_full, float *y, unsigned phases, void *ws, size_t ws_bytes, void *stream) {
  return layer_fwd(s, w, x, k_full, v_full, y, nullptr, nullptr, nullptr, phases, ws, ws_bytes, stream);
}

tsp_status tsp_layer_fwd_save(const tsp_shape *s, const tsp_layer_weights *w, const float *x, void *k_full,
                              void *v_full, float *y, float *o_save, float *lse_save, void *z_save, unsigned phases,
                              void *ws, size_t ws_bytes, void *stream) {
  if (!o_save) return fail(TSP_ERR_INVALID_ARG, "o_save is NULL");
  if (!lse_save) return fail(TSP_ERR_INVALID_ARG, "lse_save is NULL");
  return layer_fwd(s, w, x, k_full, v_full, y, o_save, lse_save, z_save, phases, ws, ws_bytes, stream);
}

// The layer backward; with o_saved and lse_saved (bf16, from
// tsp_layer_fwd_save), the attention forward is not run again: Q is
// recomputed pre-scaled, as the forward had it, and the attention backward
// takes the saved output and statistics.
static tsp_status layer_bwd(const tsp_shape *s, const tsp_layer_weights *w, const float *x, const void *k_full,
                            const void *v_full, const float *dy, const float *o_saved, const float *lse_saved,
                            const void *z_saved, float *dk_full, float *dv_full, const float *dk_loc, const float *dv_loc, float *dx,
                            const tsp_layer_grads *gr, unsigned phases, void *ws_, size_t ws_bytes, void *stream_) {
  tsp_status st = check_layer_bwd_shape(s);
  if (st) return st;
  const bool saved = o_saved != nullptr || lse_saved != nullptr;
  if (saved && (!o_saved || !lse_saved)) return fail(TSP_ERR_INVALID_ARG, "o_saved and lse_saved must both be given");
  if (saved && s->dtype != TSP_BF16) return fail(TSP_ERR_UNSUPPORTED, "the saved attention output needs bf16");
  if (saved && ((st = check_ptr(o_saved, "o_saved")) || (st = check_ptr(lse_saved, "lse_saved")))) return st;
  if (z_saved) {
    if (!saved) return fail(TSP_ERR_INVALID_ARG, "z_saved needs o_saved and lse_saved");
    if ((st = check_ptr(z_saved, "z_saved"))) return st;
  }
  if (!w) return fail(TSP_ERR_INVALID_ARG, "weights is NULL");
  if (!gr) return fail(TSP_ERR_INVALID_ARG, "grads is NULL");
  if (phases == 0 || (phases & ~3u)) return fail(TSP_ERR_INVALID_ARG, "phases=%u must be 1, 2 or 3", phases);
  if (phases == TSP_BWD_ALL && s->D != 1)
    return fail(TSP_ERR_INVALID_ARG, "TSP_BWD_ALL needs D=1 (D=%d ranks exchange K/V gradients between the phases)",
                s->D);
  const bool pa = (phases & TSP_BWD_ATTN) != 0, pq = (phases & TSP_BWD_QKV) != 0;
  const int32_t N = (int32_t)(s->S / s->D), h = s->h, D = s->D, hd = h / D, fd = s->F / D;
  const int32_t Hkv = kv_heads(s), hkv = Hkv * s->Dh, hq = h / D, hk = hkv / D, K3 = h + 2 * hkv;
  if ((st = check_ptr(x, "x")) || (st = check_ptr(ws_, "ws")) || (st = check_ptr(w->g_attn, "g_attn")) ||
      (st = check_ptr_list(w->wqkv, D, "wqkv")))
    return st;
  if (pa && ((st = check_ptr(k_full, "k_full")) || (st = check_ptr(v_full, "v_full")) || (st = check_ptr(dy, "dy")) ||
             (st = check_ptr(dk_full, "dk_full")) || (st = check_ptr(dv_full, "dv_full")) ||
             (st = check_ptr(w->g_mlp, "g_mlp")) || (st = check_ptr_list(w->wo, D, "wo")) ||
             (st = check_ptr_list(w->w1, D, "w1")) || (st = check_ptr_list(w->w2, D, "w2")) ||
             (st = check_ptr(gr->g_mlp, "grads->g_mlp")) ||
             (st = check_ptr_list((const void *const *)gr->wo, D, "grads->wo")) ||
             (st = check_ptr_list((const void *const *)gr->w1, D, "grads->w1")) ||
             (st = check_ptr_list((const void *const *)gr->w2, D, "grads->w2"))))
    return st;
  if (pq && ((st = check_ptr(dk_loc, "dk_loc")) || (st = check_ptr(dv_loc, "dv_loc")) || (st = check_ptr(dx, "dx")) ||
             (st = check_ptr(gr->g_attn, "grads->g_attn")) ||
             (st = check_ptr_list((const void *const *)gr->wqkv, D, "grads->wqkv"))))
    return st;
  const LayerBwdWs L = layer_bwd_ws(s);
  if (ws_bytes < L.total) return fail(TSP_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, L.total);
  const size_t e = elem_bytes(s->dtype), nh4 = (size_t)N * h * 4, kvf = (size_t)s->S * hkv;
  // what the requested phases read and write; dk_loc/dv_loc may be
  // dk_full/dv_full themselves when both phases run (D = 1)
  std::vector<Range> in, out;
  in.push_back({x, nh4, "x"});
  in.push_back({w->g_attn, (size_t)h * e, "g_attn"});
  for (int j = 0; j < D; ++j) in.push_back({w->wqkv[j], (size_t)(hq + 2 * hk) * h * e, "wqkv"});
  out.push_back({ws_, L.total, "ws"});
  if (pa) {
    in.push_back({k_full, kvf * e, "k_full"});
    in.push_back({v_full, kvf * e, "v_full"});
    in.push_back({dy, nh4, "dy"});
    in.push_back({w->g_mlp, (size_t)h * e, "g_mlp"});
    if (saved) {
      in.push_back({o_saved, nh4, "o_saved"});
      in.push_back({lse_saved, (size_t)s->H * N * 4, "lse_saved"});
    }
    if (z_saved) in.push_back({z_saved, (size_t)N * s->F * 2, "z_saved"});
    out.push_back({dk_full, kvf * 4, "dk_full"});
    out.push_back({dv_full, kvf * 4, "dv_full"});
    out.push_back({gr->g_mlp, (size_t)h * 4, "grads->g_mlp"});
    for (int j = 0; j < D; ++j) {
      in.push_back({w->wo[j], (size_t)h * hd * e, "wo"});
      in.push_back({w->w1[j], (size_t)fd * h * e, "w1"});
      in.push_back({w->w2[j], (size_t)h * fd * e, "w2"});
      out.push_back({gr->wo[j], (size_t)h * hd * 4, "grads->wo"});
      out.push_back({gr->w1[j], (size_t)fd * h * 4, "grads->w1"});
      out.push_back({gr->w2[j], (size_t)h * fd * 4, "grads->w2"});
    }
  }
  if (pq) {
    const bool same_k = pa && (const void *)dk_loc == (const void *)dk_full;
    const bool same_v = pa && (const void *)dv_loc == (const void *)dv_full;
    if (!same_k) in.push_back({dk_loc, (size_t)N * hkv * 4, "dk_loc"});
    if (!same_v) in.push_back({dv_loc, (size_t)N * hkv * 4, "dv_loc"});
    out.push_back({dx, nh4, "dx"});
    out.push_back({gr->g_attn, (size_t)h * 4, "grads->g_attn"});
    for (int j = 0; j < D; ++j) out.push_back({gr->wqkv[j], (size_t)(hq + 2 * hk) * h * 4, "grads->wqkv"});
  }
  for (size_t i = 0; i < out.size(); ++i) {
    for (const Range &ri : in)
      if (overlap(out[i], ri)) return fail(TSP_ERR_INVALID_ARG, "%s overlaps %s", out[i].name, ri.name);
    for (size_t j = i + 1; j < out.size(); ++j)
      if (overlap(out[i], out[j])) return fail(TSP_ERR_INVALID_ARG, "%s overlaps %s", out[i].name, out[j].name);
  }

  unsigned char *ws = static_cast<unsigned char *>(ws_);
  float *dh1 = (float *)(ws + L.dh1), *dq = (float *)(ws + L.dq);
  const tsp::ZigzagMap zz = tsp::make_zigzag(s->S, D, s->r);
  const int dt = s->dtype;
  const bool pnl = dt == TSP_BF16;  // bf16 A operands in panel layout
  const int64_t np = pnl ? (int64_t)N * tsp::kPanel : 0;
  hipStream_t stream = (hipStream_t)stream_;
  auto one = [](const void *p) {
    tsp::PtrList l;
    memset(&l, 0, sizeof l);
    l.p[0] = p;
    return l;
  };
  if (pa) {
    void *xn = ws + L.xn, *q = ws + L.q, *olo = ws + L.olo, *ot = ws + L.ot, *hn = ws + L.hn, *dylo = ws + L.dylo;
    void *dh1lo = ws + L.dh1lo, *dh1t = ws + L.dh1t, *wot = ws + L.wot, *dout = ws + L.dout;
    float *o = (float *)(ws + L.o), *h1 = (float *)(ws + L.h1), *dhn = (float *)(ws + L.dhn);
    float *lse = (float *)(ws + L.lse), *part = (float *)(ws + L.part);
    float *stat_lse = (float *)(ws + L.stat), *stat_delta = (float *)(ws + L.stat + attn_bwd_ws(s) / 2);
    // the rank's forward again: xn, Q, o with its row statistics (or the
    // saved ones), h1, hn. With the saved statistics Q is recomputed with
    // the forward's pre-scaling, which gives the forward's Q bit for bit
    // (the same inputs, the same reduction order for every element, the
    // same epilogue), so the saved statistics belong to it.
    const float q_scale = saved ? s->scale * 1.4426950408889634f : 1.0f;
    TSP_LAUNCH(TSP_K_RMSNORM, tsp::launch_rmsnorm(x, w->g_attn, xn, N, h, s->eps, dt, pnl, stream), "RMSNorm");
    TSP_LAUNCH(TSP_K_QKV,
               tsp::launch_qkv(dt, xn, pnl, N, h, to_list(w->wqkv, D), D, hq, 0, q, nullptr, nullptr, zz, q_scale,
                               nullptr, s->Dh, stream),
               "Q");
    const float *o_in = saved ? o_saved : o, *lse_in = saved ? lse_saved : lse;
    if (!saved)
      TSP_LAUNCH(TSP_K_ATTN,
                 tsp::launch_attention(dt, q, k_full, v_full, o, TSP_F32, false, s->S, N, s->H, Hkv, s->Dh, s->scale,
                                       zz, false, stream, pnl ? lse : nullptr),
                 "attention");
    TSP_LAUNCH(TSP_K_ROWS_BWD, tsp::launch_pack_cols(dt, o_in, nullptr, nullptr, N, 1, h, 0, olo, pnl, stream),
               "o conversion");
    TSP_LAUNCH(TSP_K_OUTPROJ, tsp::launch_outproj(dt, olo, pnl, N, h, to_list(w->wo, D), D, hd, x, h1, stream),
               "output projection");
    TSP_LAUNCH(TSP_K_RMSNORM, tsp::launch_rmsnorm(h1, w->g_mlp, hn, N, h, s->eps, dt, false, stream), "RMSNorm");
    // MLP branch: dhn, and the ring shards' dW1, dW2 (Z from the forward when kept)
    TSP_LAUNCH(TSP_K_ROWS_BWD, tsp::launch_pack_cols(dt, dy, nullptr, nullptr, N, 1, h, 0, dylo, false, stream),
               "dy conversion");
    if ((st = mlp_ring_bwd(s, hn, z_saved, w->w1, w->w2, dylo, nullptr, dhn, gr->w1, gr->w2, ws + L.mlp,
                           L.mlp_bytes, stream_)))
      return st;
    // dh1 = dy + the second RMSNorm's backward of dhn
    TSP_LAUNCH(TSP_K_ROWS_BWD,
               tsp::launch_rmsnorm_bwd(h1, w->g_mlp, dhn, dy, dh1, dh1lo, pnl, N, h, s->eps, dt, part, gr->g_mlp,
                                       stream),
               "RMSNorm backward");
    // output projection: do = dh1 W_O (W_O^T stacked by shard), dW_O,j =
    // dh1^T o[:, head group j]
    TSP_LAUNCH(TSP_K_TRANSPOSE,
               tsp::launch_transpose(dt, to_list(w->wo, D), D, hd, 0, h, hd, wot, h, 0, (int64_t)hd * h, stream),
               "W_O transpose");
    TSP_LAUNCH(TSP_K_BWD_GEMM, tsp::launch_gemm_nt(dt, dh1lo, pnl, N, h, wot, h, dout, dt, stream), "do");
    TSP_LAUNCH(TSP_K_TRANSPOSE,
               tsp::launch_transpose(dt, one(dh1lo), 1, h, np, N, h, dh1t, N, pnl ? (int64_t)h * tsp::kPanel : 0, 0,
                                     stream),
               "dh1 transpose");
    TSP_LAUNCH(TSP_K_TRANSPOSE, tsp::launch_transpose(dt, one(olo), 1, h, np, N, h, ot, N, 0, 0, stream),
               "o transpose");
    TSP_LAUNCH(TSP_K_BWD_GEMM,
               tsp::launch_wgrad(dt, dh1t, pnl, h, ot, h, N, to_list((const void *const *)gr->wo, D), hd, false,
                                 stream),
               "dW_O");
    // attention: dq (kept for the second phase) and this rank's share of
    // every key/value row's gradient
    TSP_LAUNCH(TSP_K_ATTN_BWD,
               tsp::launch_attention_bwd(dt, q, k_full, v_full, dout, dq, dk_full, dv_full, stat_lse, stat_delta, s->S,
                                         N, s->H, Hkv, s->Dh, s->scale, zz, stream, pnl ? o_in : nullptr,
                                         pnl ? lse_in : nullptr, false, saved),
               "attention backward");
  }
  if (pq) {
    void *xr = ws + L.xr, *xnt = ws + L.xnt, *dqkv = ws + L.dqkv, *dqkvt = ws + L.dqkvt, *wqkvt = ws + L.wqkvt;
    float *dxn = (float *)(ws + L.dxn), *part = (float *)(ws + L.part2);
    TSP_LAUNCH(TSP_K_RMSNORM, tsp::launch_rmsnorm(x, w->g_attn, xr, N, h, s->eps, dt, false, stream), "RMSNorm");
    TSP_LAUNCH(TSP_K_TRANSPOSE, tsp::launch_transpose(dt, one(xr), 1, h, 0, N, h, xnt, N, 0, 0, stream),
               "xn transpose");
    // [dq_j | dk_j | dv_j] side by side in shard order, as the rows of W_QKV,j
    TSP_LAUNCH(TSP_K_ROWS_BWD, tsp::launch_pack_cols(dt, dq, dk_loc, dv_loc, N, D, hq, hk, dqkv, pnl, stream),
               "dQKV packing");
    TSP_LAUNCH(TSP_K_TRANSPOSE,
               tsp::launch_transpose(dt, one(dqkv), 1, K3, np, N, K3, dqkvt, N, pnl ? (int64_t)K3 * tsp::kPanel : 0, 0,
                                     stream),
               "dQKV transpose");
    TSP_LAUNCH(TSP_K_TRANSPOSE,
               tsp::launch_transpose(dt, to_list(w->wqkv, D), D, h, 0, hq + 2 * hk, h, wqkvt, K3, 0, hq + 2 * hk,
                                     stream),
               "W_QKV transpose");
    TSP_LAUNCH(TSP_K_BWD_GEMM, tsp::launch_gemm_nt(dt, dqkv, pnl, N, K3, wqkvt, h, dxn, TSP_F32, stream), "dxn");
    TSP_LAUNCH(TSP_K_BWD_GEMM,
               tsp::launch_wgrad(dt, dqkvt, pnl, K3, xnt, h, N, to_list((const void *const *)gr->wqkv, D), hq + 2 * hk,
                                 true, stream),
               "dW_QKV");
    TSP_LAUNCH(TSP_K_ROWS_BWD,
               tsp::launch_rmsnorm_bwd(x, w->g_attn, dxn, dh1, dx, nullptr, false, N, h, s->eps, dt, part, gr->g_attn,
                                       stream),
               "RMSNorm backward");
  }
  return ok();
}

tsp_status tsp_layer_bwd(const tsp_shape *s, const tsp_layer_weights *w, const float *x, const void *k_full,
                         const void *v_full, const float *dy, float *dk_full, float *dv_full, const float *dk_loc,
                         const float *dv_loc, float *dx, const tsp_layer_grads *gr, unsigned phases, void *ws,
                         size_t ws_bytes, void *stream) {
  return layer_bwd(s, w, x, k_full, v_full, dy, nullptr, nullptr, nullptr, dk_full, dv_full, dk_loc, dv_loc, dx, gr,
                   phases, ws, ws_bytes, stream);
}

tsp_status tsp_layer_bwd_ex(const tsp_shape *s, const tsp_layer_weights *w, const float *x, const void *k_full,
                            const void *v_full, const float *dy, const float *o_saved, const float *lse_saved,
                            const void *z_saved, float *dk_full, float *dv_full, const float *dk_loc,
                            const float *dv_loc, float *dx, const tsp_layer_grads *gr, unsigned phases, void *ws,
                            size_t ws_bytes, void *stream) {
  return layer_bwd(s, w, x, k_full, v_full, dy, o_saved, lse_saved, z_saved, dk_full, dv_full, dk_loc, dv_loc, dx, gr,
                   phases, ws, ws_bytes, stream);
}

void tsp_profile_enable(int on) { g_prof.on = on != 0; }

void tsp_profile_reset(void) {
  for (int k = 0; k < TSP_K_COUNT; ++k) {
    g_prof.drain(k);
    g_prof.ms[k] = 0.0;
    g_prof.n[k] = 0;
  }
}

tsp_status tsp_profile_read(int k, double *total_ms, int64_t *launches) {
  if (k < 0 || k >= TSP_K_COUNT) return fail(TSP_ERR_INVALID_ARG, "unknown kernel class %d", k);
  if (!total_ms || !launches) return fail(TSP_ERR_INVALID_ARG, "output pointer is NULL");
  g_prof.drain(k);
  *total_ms = g_prof.ms[k];
  *launches = g_prof.n[k];
  return ok();
}

}  // extern "C"
