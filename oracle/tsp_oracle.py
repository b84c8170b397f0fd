"""CPU oracle for one TSP decoder layer on one rank's share of the work.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or call this module. The HIP library
never uses it and shares no code with it.

Everything here is plain, unblocked numpy in float64 (scipy's erf for GELU),
written from the definitions so that it can be checked by eye.

Sources (the pages describe the method; no code was published):
  [P2] zubnet.ai news item "Zyphra TSP folds TP+SP onto one GPU axis"
       (in Hindi). Paragraph 1: one mesh axis of size D carries both weight
       and token sharding; each GPU keeps 1/D of the weights and 1/D of the
       tokens; the validated model is a 7B dense decoder (hidden 4096,
       32 layers, 32 query/KV heads, MLP 4x, bf16) at 128K tokens with D=8.
       Paragraph 2: for attention, weight shards are broadcast one after
       another and each GPU applies each to its own tokens, then K and V are
       all-gathered under a zigzag partition that balances load; for the MLP,
       weight shards travel round a ring of point-to-point transfers, so the
       all-reduce of ordinary tensor parallelism disappears.
       Paragraph 4: the MLP without all-reduce carries over to other setups.
  [P1] ageofai.tools "Zyphra TSP: 2.6x Faster AI Training Review":
       TSP merges tensor and sequence parallelism on one GPU axis (What's New).

Readings where the pages are silent (each is restated where it is used):
  R1 zigzag: the sequence is cut into 2D equal chunks; rank r owns chunks r
     and 2D-1-r, kept in that order, ascending inside each chunk.
  R2 attention shards are head groups: shard j holds heads j*H/D..(j+1)*H/D-1
     of W_Q, W_K, W_V (output rows) and of W_O (input columns).
  R3 the gathered K/V are full-sequence, all heads, in global position order.
  R4 causal mask is inclusive (key u is visible to the query at p iff u <= p),
     softmax scale 1/sqrt(Dh), no bias; rotary embedding and grouped K/V heads
     only as the optional variants R7 and R8.
  R5 the MLP is two matrices with exact (erf) GELU, width F = 4h; MLP shard j
     holds hidden units j*F/D..(j+1)*F/D-1 (rows of W1, columns of W2).
  R6 pre-RMSNorm residual block: h1 = x + Attn(RMSNorm(x)),
     y = h1 + MLP(RMSNorm(h1)); eps = 1e-5; no biases.
  R7 rotary position embedding (an optional variant; the pages' model has
     none): with rope_base > 0, Q and K of each token are rotated by its
     global position p before attention. Feature d and feature d + Dh/2 of a
     head form a pair (the rotate-half convention); pair i turns by the
     angle p * rope_base^(-2i/Dh).
  R8 grouped-query attention (an optional variant; the pages' model is
     multi-head): Hkv K/V heads, each shared by H/Hkv consecutive query heads
     (query head i reads K/V head i // (H/Hkv)); shard j then holds query
     heads j*H/D.. and K/V heads j*Hkv/D.. Hkv = H is multi-head attention.
  R9 gated MLP (an optional variant; the pages' MLP is R5): the hidden layer
     is SiLU(x W_g^T) * (x W_u^T), elementwise, with SiLU(z) = z / (1 + e^-z)
     (the SwiGLU form of common 7B models), then W_2 as in R5. Shard j holds
     hidden units j*F/D..(j+1)*F/D-1: its first matrix stacks the W_g rows of
     those units on the W_u rows of the same units, [2F/D, h].
  R10 backward of the MLP ring (an optional extension; the pages give the
     2.6x figure for training but describe only how shards move): the
     gradients are those of the unsharded branch y = GELU(x W1^T) W2^T by the
     chain rule. A rank's input gradient is summed over the shards it
     receives, again with no all-reduce; its weight gradients are its own
     tokens' contribution to each shard's gradient, and the D ranks'
     contributions add up to the gradient over the whole sequence (the sum a
     ring would carry back to the shard's owner).
  R12 backward of the whole layer (an optional extension, like R10): the
     gradients of the pre-norm layer (R6) by the chain rule, on one rank in
     two halves around the exchange that returns key/value gradients to
     their owners. First half: the rank recomputes its own forward from x,
     then takes the MLP ring backward (R10), the second RMSNorm's backward,
     the output projection's backward and the attention backward (R11); its
     K/V gradients cover every key row. Second half, once the rank holds the
     summed gradients of its own K/V rows: the QKV projection's backward and
     the first RMSNorm's backward. Weight and gain gradients are the rank's
     own tokens' contribution (the D ranks' contributions add up to the
     gradient over the whole sequence). No rotation, grouped K/V heads as in
     R8, the pages' GELU MLP only.
  R11 backward of the zigzag attention (an optional extension, like R10):
     the gradients of causal_attention by the chain rule through the
     softmax. A rank's queries give their own dQ rows; its dK and dV are its
     queries' contribution to every key row (the D ranks' contributions add
     up to the whole sequence's dK and dV, the sum that would travel back to
     each row's owner after the all-gather).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf
from scipy.special import expit as _expit

__all__ = [
    "zigzag_positions",
    "zigzag_owner",
    "rms_norm",
    "gelu",
    "silu",
    "causal_attention",
    "rope",
    "unshard_attention_weights",
    "unshard_mlp_weights",
    "mlp",
    "mlp_shard",
    "gelu_grad",
    "softmax_backward",
    "causal_attention_lse",
    "causal_attention_backward",
    "mlp_backward",
    "rms_norm_backward",
    "layer_bwd_attn_part",
    "layer_bwd_qkv_part",
    "layer_backward_full",
    "layer_full",
    "layer_rows",
    "local_kv",
    "layer_rank",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Token ownership
# --------------------------------------------------------------------------
def zigzag_positions(S: int, D: int, r: int) -> np.ndarray:
    """Global positions of the S/D tokens rank r holds, in local row order.

    [P2] paragraph 2 names a zigzag partition of the sequence for load
    balance; reading R1 fixes the rule: 2D chunks of C = S/(2D) tokens, rank
    r holds chunk r followed by chunk 2D-1-r.
    """
    if D < 1 or S % (2 * D) != 0 or not (0 <= r < D):
        raise ValueError("need D >= 1, S divisible by 2D and 0 <= r < D")
    C = S // (2 * D)
    pos = []
    for chunk in (r, 2 * D - 1 - r):
        for i in range(C):
            pos.append(chunk * C + i)
    return np.array(pos, dtype=np.int64)


def zigzag_owner(p: int, S: int, D: int):
    """(rank, local row) that holds global position p under reading R1."""
    C = S // (2 * D)
    chunk = p // C
    if chunk < D:
        return chunk, p % C
    return 2 * D - 1 - chunk, C + p % C


# --------------------------------------------------------------------------
# Layer pieces
# --------------------------------------------------------------------------
def rms_norm(x, g, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g (reading R6)."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(g)


def gelu(z) -> np.ndarray:
    """Exact GELU, z * Phi(z) = z * (1 + erf(z / sqrt 2)) / 2 (reading R5)."""
    z = _f64(z)
    return 0.5 * z * (1.0 + _erf(z / np.sqrt(2.0)))


def silu(z) -> np.ndarray:
    """SiLU, z * sigma(z) = z / (1 + e^-z) (reading R9); sigma from scipy's
    expit, which does not overflow for large |z|."""
    z = _f64(z)
    return z * _expit(z)


def causal_attention(q, k, v, q_pos, scale: float, row_block: int = 256) -> np.ndarray:
    """Softmax attention of queries at global positions q_pos over K/V.

    q: [n, H, Dh] queries; k, v: [S, Hkv, Dh] full-sequence keys and values
    in global order (reading R3, the result of the all-gather in [P2]
    paragraph 2), Hkv dividing H (query head i reads K/V head i // (H/Hkv),
    reading R8); q_pos: [n] global position of each query. For each query t
    and head, the scores scale * <q, k_u> over keys u <= q_pos[t] (reading R4)
    go through a softmax that weights the values.

    Rows are taken row_block at a time to bound memory; each row is computed
    independently and in full, with its own softmax over its whole prefix.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n, H, Dh = q.shape
    group = H // k.shape[1]
    out = np.empty((n, H, Dh), dtype=np.float64)
    for lo in range(0, n, row_block):
        hi = min(n, lo + row_block)
        pos = q_pos[lo:hi]
        L = int(pos.max()) + 1
        visible = np.arange(L)[None, :] <= pos[:, None]
        for hd in range(H):
            qh = _f64(q[lo:hi, hd, :])
            kh = _f64(k[:L, hd // group, :])
            vh = _f64(v[:L, hd // group, :])
            s = scale * (qh @ kh.T)
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[lo:hi, hd, :] = p @ vh
    return out


def causal_attention_lse(q, k, q_pos, scale: float, row_block: int = 256) -> np.ndarray:
    """Natural log of each row's softmax denominator in causal_attention,
    log sum_{u <= q_pos[t]} exp(scale * <q, k_u>), as [H, n] (reading R11:
    the row statistic a backward can take from its forward). Evaluated as
    max + log(sum(exp(s - max))), which is the same number without overflow."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n, H, _ = q.shape
    group = H // k.shape[1]
    out = np.empty((H, n), dtype=np.float64)
    for lo in range(0, n, row_block):
        hi = min(n, lo + row_block)
        pos = q_pos[lo:hi]
        L = int(pos.max()) + 1
        visible = np.arange(L)[None, :] <= pos[:, None]
        for hd in range(H):
            s = np.where(visible, scale * (_f64(q[lo:hi, hd, :]) @ _f64(k[:L, hd // group, :]).T), -np.inf)
            mx = s.max(axis=1)
            out[hd, lo:hi] = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    return out


def softmax_backward(p, dp) -> np.ndarray:
    """Gradient of the scores from that of the probabilities, row by row: the
    Jacobian of softmax gives ds_u = p_u * (dp_u - sum_w p_w dp_w) (R11)."""
    p, dp = _f64(p), _f64(dp)
    return p * (dp - (p * dp).sum(axis=-1, keepdims=True))


def causal_attention_backward(q, k, v, q_pos, scale: float, do, row_block: int = 256) -> dict:
    """Gradients of causal_attention (reading R11) for an output gradient do
    [n, H, Dh]: dq [n, H, Dh] and dk, dv [S, Hkv, Dh].

    Per query t and head, with s_u = scale * <q, k_u> over the visible keys
    u <= q_pos[t], p = softmax(s) and o = sum_u p_u v_u: dp_u = <do, v_u>,
    the softmax Jacobian gives ds_u = p_u * (dp_u - sum_w p_w dp_w), and then
    dq = scale * sum_u ds_u k_u, dk_u += scale * ds_u q, dv_u += p_u do. Rows
    are taken row_block at a time, each with its whole prefix; K/V head i //
    (H/Hkv) collects the gradients of every query head that reads it (R8).
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n, H, Dh = q.shape
    Skv, Hkv = k.shape[0], k.shape[1]
    group = H // Hkv
    dq = np.zeros((n, H, Dh), dtype=np.float64)
    dk = np.zeros((Skv, Hkv, Dh), dtype=np.float64)
    dv = np.zeros((Skv, Hkv, Dh), dtype=np.float64)
    for lo in range(0, n, row_block):
        hi = min(n, lo + row_block)
        pos = q_pos[lo:hi]
        L = int(pos.max()) + 1
        visible = np.arange(L)[None, :] <= pos[:, None]
        for hd in range(H):
            kv = hd // group
            qh = _f64(q[lo:hi, hd, :])
            kh = _f64(k[:L, kv, :])
            vh = _f64(v[:L, kv, :])
            doh = _f64(do[lo:hi, hd, :])
            s = np.where(visible, scale * (qh @ kh.T), -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p = p / p.sum(axis=1, keepdims=True)
            ds = softmax_backward(p, doh @ vh.T)
            dq[lo:hi, hd, :] = scale * (ds @ kh)
            dk[:L, kv, :] += scale * (ds.T @ qh)
            dv[:L, kv, :] += p.T @ doh
    return {"dq": dq, "dk": dk, "dv": dv}


def rope(x, pos, base: float) -> np.ndarray:
    """Rotary position embedding of x [n, H, Dh] at global positions pos [n]
    (reading R7). base <= 0 leaves x unchanged.

    Pair i (0 <= i < Dh/2) is features (i, i + Dh/2); it turns by the angle
    pos * base^(-2i/Dh): (a, b) -> (a cos - b sin, b cos + a sin).
    """
    x = _f64(x)
    if base <= 0:
        return x
    half = x.shape[-1] // 2
    inv_freq = float(base) ** (-2.0 * np.arange(half, dtype=np.float64) / x.shape[-1])
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]  # [n, half]
    cos, sin = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


# --------------------------------------------------------------------------
# Shards -> unsharded matrices
# --------------------------------------------------------------------------
def unshard_attention_weights(wqkv, wo, H: int, Dh: int, Hkv: int | None = None):
    """Rebuild W_Q [H*Dh, h], W_K, W_V [Hkv*Dh, h] and W_O [h, H*Dh] (out, in)
    from the D shards.

    Reading R2: shard j's rows are the Q rows, then K rows, then V rows of its
    head group (H/D query heads, Hkv/D K/V heads, reading R8), so
    concatenating shard j's Q rows over j in order gives W_Q, and W_O is the
    concatenation of the shards' columns.
    """
    D = len(wqkv)
    Hkv = H if Hkv is None else Hkv
    hq, hkv = (H // D) * Dh, (Hkv // D) * Dh
    wq = np.concatenate([_f64(w)[0:hq] for w in wqkv], axis=0)
    wk = np.concatenate([_f64(w)[hq:hq + hkv] for w in wqkv], axis=0)
    wv = np.concatenate([_f64(w)[hq + hkv:hq + 2 * hkv] for w in wqkv], axis=0)
    w_o = np.concatenate([_f64(w) for w in wo], axis=1)
    return wq, wk, wv, w_o


def unshard_mlp_weights(w1, w2, gated: bool = False):
    """Rebuild W1 [F, h] and W2 [h, F] (out, in) from the D shards (reading
    R5). gated: returns W_g, W_u [F, h] and W2 instead (reading R9: shard j's
    first matrix is its W_g rows above its W_u rows)."""
    W2 = np.concatenate([_f64(w) for w in w2], axis=1)
    if not gated:
        return np.concatenate([_f64(w) for w in w1], axis=0), W2
    halves = [np.split(_f64(w), 2, axis=0) for w in w1]
    return np.concatenate([g for g, _ in halves], axis=0), np.concatenate([u for _, u in halves], axis=0), W2


# --------------------------------------------------------------------------
# MLP
# --------------------------------------------------------------------------
def mlp(x, w1, w2, gated: bool = False) -> np.ndarray:
    """Unsharded MLP branch GELU(x W1^T) W2^T from lists of shards (reading
    R5), or with gated, (SiLU(x W_g^T) * (x W_u^T)) W2^T (reading R9).

    [P2] paragraphs 2 and 4: the ring applies each shard to the local tokens
    and sums the contributions without an all-reduce; this is the unsharded
    quantity that sum must equal.
    """
    x = _f64(x)
    if gated:
        Wg, Wu, W2 = unshard_mlp_weights(w1, w2, gated=True)
        return (silu(x @ Wg.T) * (x @ Wu.T)) @ W2.T
    W1, W2 = unshard_mlp_weights(w1, w2)
    return gelu(x @ W1.T) @ W2.T


def mlp_shard(x, w1_j, w2_j, gated: bool = False) -> np.ndarray:
    """One shard's contribution GELU(x W1_j^T) W2_j^T (reading R5), or the
    gated form of reading R9."""
    x = _f64(x)
    if gated:
        wg, wu = np.split(_f64(w1_j), 2, axis=0)
        return (silu(x @ wg.T) * (x @ wu.T)) @ _f64(w2_j).T
    return gelu(x @ _f64(w1_j).T) @ _f64(w2_j).T


# --------------------------------------------------------------------------
# MLP backward (reading R10)
# --------------------------------------------------------------------------
def gelu_grad(z) -> np.ndarray:
    """Derivative of the exact GELU (reading R5): Phi(z) + z * phi(z), with
    phi(z) = exp(-z^2/2) / sqrt(2 pi) the standard normal density."""
    z = _f64(z)
    cdf = 0.5 * (1.0 + _erf(z / np.sqrt(2.0)))
    pdf = np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)
    return cdf + z * pdf


def mlp_backward(x, w1, w2, dy) -> dict:
    """Gradients of the MLP branch y = GELU(x W1^T) W2^T (readings R5, R10).

    x: [n, h] branch input (the normalised tokens), w1/w2: the D shards
    ([F/D, h] rows of W1, [h, F/D] columns of W2), dy: [n, h] gradient of the
    branch output. With Z = x W1^T and H = GELU(Z), the chain rule gives
    dH = dy W2, dZ = dH * GELU'(Z), dx = dZ W1, dW1 = dZ^T x, dW2 = dy^T H.
    Returns dx [n, h] and the shard slices of dW1 and dW2 as lists indexed by
    shard (the same split as the weights). Evaluated on a rank's own tokens
    this is that rank's contribution to each shard's gradient.
    """
    x, dy = _f64(x), _f64(dy)
    W1, W2 = unshard_mlp_weights(w1, w2)
    Z = x @ W1.T
    H = gelu(Z)
    dZ = (dy @ W2) * gelu_grad(Z)
    dW1 = dZ.T @ x
    dW2 = dy.T @ H
    fd = W1.shape[0] // len(w1)
    return {
        "dx": dZ @ W1,
        "dw1": [dW1[j * fd:(j + 1) * fd] for j in range(len(w1))],
        "dw2": [dW2[:, j * fd:(j + 1) * fd] for j in range(len(w2))],
    }


# --------------------------------------------------------------------------
# Layer backward (reading R12)
# --------------------------------------------------------------------------
def rms_norm_backward(x, g, eps: float, dout):
    """Gradients of rms_norm (R6) for an output gradient dout, row by row.
    With r = (mean(x^2) + eps)^(-1/2) and y_i = g_i x_i r, the derivative of
    r is -r^3 x_k / h, so dx_k = r g_k dout_k - (r^3 x_k / h) sum_i dout_i
    g_i x_i, and dg_i = sum over rows of dout_i x_i r. Returns (dx, dg)."""
    x, g, dout = _f64(x), _f64(g), _f64(dout)
    h = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    dx = r * g * dout - (r ** 3) * x * np.sum(dout * g * x, axis=-1, keepdims=True) / h
    dg = np.sum(dout * x * r, axis=0)
    return dx, dg


def layer_bwd_attn_part(x_local, pos, w: dict, k_full, v_full, dy, H: int, Dh: int, eps: float, scale: float,
                        Hkv: int | None = None) -> dict:
    """First half of a rank's layer backward (reading R12).

    x_local: [n, h] the rank's tokens, pos: [n] their global positions,
    k_full, v_full: [S, Hkv, Dh] the gathered K/V (the rank's own rows
    included), dy: [n, h] gradient of the layer output. The rank's forward is
    recomputed (xn, q, o, h1, hn); then, in reverse: the MLP branch
    (mlp_backward on hn), the second RMSNorm (dh1 = dy + its backward), the
    output projection (do = dh1 W_O, dW_O = dh1^T o), the attention
    (causal_attention_backward). Returns dh1, dq [n, H, Dh], dk, dv
    [S, Hkv, Dh] (this rank's contribution to every key row), dwo, dw1, dw2
    (shard lists, this rank's contribution), dg_mlp, and the recomputed xn.
    """
    x = _f64(x_local)
    n, h = x.shape
    Hkv = H if Hkv is None else Hkv
    wq, _, _, w_o = unshard_attention_weights(w["wqkv"], w["wo"], H, Dh, Hkv)
    xn = rms_norm(x, w["g_attn"], eps)
    q = (xn @ wq.T).reshape(n, H, Dh)
    o = causal_attention(q, k_full, v_full, pos, scale)
    o2 = o.reshape(n, H * Dh)
    h1 = x + o2 @ w_o.T
    hn = rms_norm(h1, w["g_mlp"], eps)
    mb = mlp_backward(hn, w["w1"], w["w2"], dy)
    dhn_h1, dg_mlp = rms_norm_backward(h1, w["g_mlp"], eps, mb["dx"])
    dh1 = _f64(dy) + dhn_h1
    do = dh1 @ w_o
    dWo = dh1.T @ o2
    hd = w_o.shape[1] // len(w["wo"])
    ab = causal_attention_backward(q, k_full, v_full, pos, scale, do.reshape(n, H, Dh))
    return {"dh1": dh1, "dq": ab["dq"], "dk": ab["dk"], "dv": ab["dv"],
            "dwo": [dWo[:, j * hd:(j + 1) * hd] for j in range(len(w["wo"]))],
            "dw1": mb["dw1"], "dw2": mb["dw2"], "dg_mlp": dg_mlp, "xn": xn, "h1": h1}


def layer_bwd_qkv_part(x_local, w: dict, dh1, dq, dk_loc, dv_loc, H: int, Dh: int, eps: float,
                       Hkv: int | None = None) -> dict:
    """Second half of a rank's layer backward (reading R12), once the rank
    holds the summed gradients dk_loc, dv_loc [n, Hkv, Dh] of its own K/V
    rows. With xn = RMSNorm(x) recomputed: dxn = dq W_Q + dk W_K + dv W_V,
    each shard's gradient dW_QKV,j = [dq_j | dk_j | dv_j]^T xn (its Q, K and V
    rows, as in the weights' layout), and dx = dh1 + the first RMSNorm's
    backward of dxn. Returns dx [n, h], dwqkv (shard list, this rank's
    contribution) and dg_attn."""
    x = _f64(x_local)
    n, h = x.shape
    Hkv = H if Hkv is None else Hkv
    D = len(w["wqkv"])
    wq, wk, wv, _ = unshard_attention_weights(w["wqkv"], w["wo"], H, Dh, Hkv)
    xn = rms_norm(x, w["g_attn"], eps)
    dq2, dk2, dv2 = _f64(dq).reshape(n, H * Dh), _f64(dk_loc).reshape(n, Hkv * Dh), _f64(dv_loc).reshape(n, Hkv * Dh)
    dxn = dq2 @ wq + dk2 @ wk + dv2 @ wv
    hq, hk = (H // D) * Dh, (Hkv // D) * Dh
    dwqkv = [np.concatenate([dq2[:, j * hq:(j + 1) * hq].T @ xn, dk2[:, j * hk:(j + 1) * hk].T @ xn,
                             dv2[:, j * hk:(j + 1) * hk].T @ xn], axis=0) for j in range(D)]
    dx_n, dg_attn = rms_norm_backward(x, w["g_attn"], eps, dxn)
    return {"dx": _f64(dh1) + dx_n, "dwqkv": dwqkv, "dg_attn": dg_attn}


def layer_backward_full(x, w: dict, dy, H: int, Dh: int, eps: float, scale: float, Hkv: int | None = None) -> dict:
    """Backward of the unsharded layer over the whole sequence (reading R12
    with one rank: its K/V rows are all the rows, so the first half's K/V
    gradients are already the full ones). x, dy: [S, h] in global order.
    Returns dx, dwqkv, dwo, dw1, dw2 (shard lists) and dg_attn, dg_mlp."""
    x = _f64(x)
    S, h = x.shape
    Hkv = H if Hkv is None else Hkv
    _, wk, wv, _ = unshard_attention_weights(w["wqkv"], w["wo"], H, Dh, Hkv)
    pos = np.arange(S)
    xn = rms_norm(x, w["g_attn"], eps)
    k = (xn @ wk.T).reshape(S, Hkv, Dh)
    v = (xn @ wv.T).reshape(S, Hkv, Dh)
    a = layer_bwd_attn_part(x, pos, w, k, v, dy, H, Dh, eps, scale, Hkv)
    b = layer_bwd_qkv_part(x, w, a["dh1"], a["dq"], a["dk"], a["dv"], H, Dh, eps, Hkv)
    return {"dx": b["dx"], "dwqkv": b["dwqkv"], "dwo": a["dwo"], "dw1": a["dw1"], "dw2": a["dw2"],
            "dg_attn": b["dg_attn"], "dg_mlp": a["dg_mlp"]}


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def layer_full(x, w: dict, H: int, Dh: int, eps: float, scale: float, rope_base: float = 0.0,
               Hkv: int | None = None, gated: bool = False) -> dict:
    """Unsharded pre-norm decoder layer over the whole sequence (reading R6).

    x: [S, h] in global order. w: the shard lists wqkv, wo, w1, w2 and gains
    g_attn, g_mlp. TSP rearranges this computation over ranks and shards but
    reaches the same values ([P2] paragraphs 1-2), so this is what every rank
    must reproduce for its own rows. rope_base > 0 rotates Q and K (reading
    R7); Hkv < H groups the K/V heads (R8); gated selects the gated MLP (R9).
    Returns y and the intermediates h1, q, k, v, o.
    """
    x = _f64(x)
    S = x.shape[0]
    Hkv = H if Hkv is None else Hkv
    wq, wk, wv, w_o = unshard_attention_weights(w["wqkv"], w["wo"], H, Dh, Hkv)
    a = rms_norm(x, w["g_attn"], eps)
    q = rope((a @ wq.T).reshape(S, H, Dh), np.arange(S), rope_base)
    k = rope((a @ wk.T).reshape(S, Hkv, Dh), np.arange(S), rope_base)
    v = (a @ wv.T).reshape(S, Hkv, Dh)
    o = causal_attention(q, k, v, np.arange(S), scale)
    h1 = x + o.reshape(S, H * Dh) @ w_o.T
    m = rms_norm(h1, w["g_mlp"], eps)
    y = h1 + mlp(m, w["w1"], w["w2"], gated)
    return {"y": y, "h1": h1, "q": q, "k": k, "v": v, "o": o}


def layer_rows(x_rows, pos_rows, w: dict, k_all, v_all, H: int, Dh: int, eps: float, scale: float,
               rope_base: float = 0.0, Hkv: int | None = None, gated: bool = False) -> dict:
    """Layer output for given token rows once the full K/V are gathered (R6).

    x_rows: [m, h] tokens, pos_rows: [m] their global positions, k_all, v_all:
    [S, H, Dh] the complete gathered K/V (including these tokens' own rows).
    Every row is independent of the others here: RMSNorm, its query, its
    causal attention, the output projection, RMSNorm and the MLP. With
    rope_base > 0 the query is rotated at its position (k_all holds rotated
    keys, reading R7); gated selects the gated MLP (R9).
    """
    x_rows = _f64(x_rows)
    m = x_rows.shape[0]
    wq, _, _, w_o = unshard_attention_weights(w["wqkv"], w["wo"], H, Dh, Hkv)
    a = rms_norm(x_rows, w["g_attn"], eps)
    q = rope((a @ wq.T).reshape(m, H, Dh), pos_rows, rope_base)
    o = causal_attention(q, k_all, v_all, pos_rows, scale)
    h1 = x_rows + o.reshape(m, H * Dh) @ w_o.T
    mm = rms_norm(h1, w["g_mlp"], eps)
    y = h1 + mlp(mm, w["w1"], w["w2"], gated)
    return {"y": y, "h1": h1}


def local_kv(x_local, w: dict, H: int, Dh: int, eps: float, pos=None, rope_base: float = 0.0,
             Hkv: int | None = None):
    """K and V [n, Hkv, Dh] of a rank's own tokens (R2, R6, R8); with
    rope_base > 0 K is rotated at the tokens' global positions pos (R7)."""
    x_local = _f64(x_local)
    n = x_local.shape[0]
    Hkv = H if Hkv is None else Hkv
    _, wk, wv, _ = unshard_attention_weights(w["wqkv"], w["wo"], H, Dh, Hkv)
    a = rms_norm(x_local, w["g_attn"], eps)
    k = (a @ wk.T).reshape(n, Hkv, Dh)
    if rope_base > 0:
        k = rope(k, pos, rope_base)
    return k, (a @ wv.T).reshape(n, Hkv, Dh)


def layer_rank(x_local, w: dict, k_full, v_full, S: int, D: int, r: int,
               H: int, Dh: int, eps: float, scale: float, rows=None, rope_base: float = 0.0,
               Hkv: int | None = None, gated: bool = False) -> dict:
    """Rank r's layer output for its S/D local tokens (reading R6).

    x_local: [S/D, h] rank r's tokens in local zigzag order (R1). k_full,
    v_full: [S, Hkv, Dh] what the all-gather delivers ([P2] paragraph 2); the
    rows at rank r's own positions are replaced by the K/V this rank computes
    from x_local, the rest are used as given. rows: optional subset of local
    rows whose output is wanted (all local rows still produce K/V, since any
    later query may attend to them). rope_base > 0 rotates Q and K (R7; the
    given remote K rows are taken as already rotated); gated selects the gated
    MLP (R9). Returns y [len(rows), h] and h1.
    """
    x_local = _f64(x_local)
    n = x_local.shape[0]
    pos = zigzag_positions(S, D, r)
    if n != pos.shape[0]:
        raise ValueError("x_local must hold S/D rows")
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    k_loc, v_loc = local_kv(x_local, w, H, Dh, eps, pos, rope_base, Hkv)
    k_all = np.array(k_full, dtype=np.float64, copy=True)
    v_all = np.array(v_full, dtype=np.float64, copy=True)
    k_all[pos] = k_loc
    v_all[pos] = v_loc
    out = layer_rows(x_local[rows], pos[rows], w, k_all, v_all, H, Dh, eps, scale, rope_base, Hkv, gated)
    out["pos"] = pos[rows]
    return out
