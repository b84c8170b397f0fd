"""Analytic device memory of one rank on a TSP folded axis.

The zubnet.ai news item "Zyphra TSP folds TP+SP onto one GPU axis" says, in
paragraph 1, that each rank keeps 1/D of the model's weights and 1/D of the
sequence's tokens, so parameter memory and activation memory both fall by
the same factor 1/D. Paragraph 2 adds the exchanges that put transient data
on a rank: the attention weight shards it receives by broadcast, the MLP
shards that reach it round the ring, and the K/V rows of the other ranks
that the zigzag all-gather delivers before attention. The same paragraph
quotes 38.8 GB per GPU for TSP at 128K tokens on one node of eight MI300X,
against 70.0 GB for plain tensor parallelism; that figure is for the pages'
own training setup, whose optimizer, recomputation policy and embedding
sizes the pages do not state, so it is context here and nothing below is
fitted to it.

This module adds up, for any shape (S, D, model widths, layer count), the
bytes one rank holds on its device while it runs the layer forward this
library implements, and optionally the extra state of mixed-precision
training under stated assumptions. It is plain host arithmetic. The
workspace sizes are derived again here from the library's buffer layout
(not read from it), so that a test can hold the two against each other;
`single_gpu_bytes` gives what a one-GPU run that keeps all D shards and the
whole gathered K/V resident allocates, which the benchmark compares with
the device allocator's own count.

Only the decoder layers are counted: the pages give no vocabulary size, so
embeddings and the output head are left out.
"""
from __future__ import annotations

import dataclasses

# workspace kinds, as in the C header
WS_MLP, WS_LAYER, WS_MLP_BWD, WS_ATTN_BWD, WS_LAYER_BWD = 0, 1, 2, 3, 4
NORM_BWD_ROWS = 16  # rows per block of the RMSNorm backward (one gain partial each)

LEAD_ROWS = 64  # rank 0's leading positions that the bf16 layer recomputes in fp32


def _align256(x: int) -> int:
    return (x + 255) & ~255


def _elem(dtype: str) -> int:
    return 2 if dtype == "bf16" else 4


@dataclasses.dataclass(frozen=True)
class Model:
    """Widths of one decoder layer, the sequence and the folded axis.

    S tokens in the sequence, D ranks on the axis, r this rank; h hidden, H
    query heads of Dh, Hkv K/V heads (0 = H), F MLP hidden units, mlp 'gelu'
    (two matrices) or 'swiglu' (gate and up rows, then the down matrix);
    layers in the model; dtype of weights and activations ('bf16' or 'f32');
    rope_base > 0 when the layer applies rotary embedding (a small table)."""

    S: int
    D: int
    h: int
    H: int
    Dh: int
    F: int
    layers: int = 1
    r: int = 0
    Hkv: int = 0
    mlp: str = "gelu"
    dtype: str = "bf16"
    rope_base: float = 0.0

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def N(self) -> int:
        return self.S // self.D

    @property
    def C(self) -> int:
        return self.S // (2 * self.D)


# ----------------------------------------------------------------- workspaces
def _lead_chunk(kseg: int) -> int:
    for c in (512, 256, 128):
        if kseg % c == 0:
            return c
    return 64


def _lead_part_bytes(m: int, h: int, F: int, D: int, gated: bool) -> int:
    """Partial sums of the leading rows' products: each K chunk of each
    product writes m rows of its output columns in fp32."""
    hd, fd = h // D, F // D
    qkv = (h // _lead_chunk(h)) * m * 3 * h
    op = (h // _lead_chunk(hd)) * m * h
    up = (h // _lead_chunk(h)) * m * (2 * F if gated else F)
    dn = (F // _lead_chunk(fd)) * m * h
    return 4 * max(qkv, op, up, dn)


def lead_rows(m: Model) -> int:
    if m.dtype != "bf16" or m.r != 0:
        return 0
    return min(LEAD_ROWS, m.C)


def workspace_bytes(m: Model, kind: int) -> int:
    """Scratch bytes of one call, from the layout of its buffers:

    WS_LAYER: Q [N][h]; the normed input, later the attention output [N][h];
      the MLP hidden layer [N][F] (all in dtype); the rotary table
      [N][Dh/2] (cos, sin) fp32 when rope_base > 0; for bf16 rank 0, the
      leading rows' fp32 buffers (seven [m][h], one [m][F]) and the partial
      sums of their products.
    WS_MLP: the hidden layer [N][F] in dtype.
    WS_MLP_BWD: W1 stacked in ring order, W1^T and W2^T ([F][h] each), x^T
      and dy^T ([h][N]), Z^T and GELU(Z)^T ([F][N]), all in dtype.
    WS_ATTN_BWD: log-sum-exp and Delta of every (head, local row), fp32.
    WS_LAYER_BWD: dh1 and dq, fp32 [N][h] each, kept between the two
      phases; then the larger of the phases' own buffers. First phase: nine
      [N][h] in dtype (normed input, Q, attention output and its transpose,
      normed h1, dy, dh1 and its transpose, do), three fp32 [N][h] (attention
      output, h1, MLP input gradient), W_O^T [h][h], the forward's
      log-sum-exp [H][N] fp32, WS_ATTN_BWD, the gain partials (one fp32 row
      of h per 16 tokens) and WS_MLP_BWD. Second phase: normed input and its
      transpose, [dq|dk|dv] and its transpose ([N][h + 2 Hkv Dh] each), its
      weights transposed [h][h + 2 Hkv Dh] (all in dtype), dxn fp32 [N][h],
      the gain partials.
    Each buffer starts on a 256-byte boundary."""
    e, N, h, F = _elem(m.dtype), m.N, m.h, m.F
    if kind == WS_MLP:
        return _align256(N * F * e)
    if kind == WS_ATTN_BWD:
        return 2 * _align256(m.H * N * 4)
    if kind == WS_MLP_BWD:
        return 3 * _align256(F * h * e) + 2 * _align256(h * N * e) + 2 * _align256(F * N * e)
    if kind == WS_LAYER_BWD:
        nh, nh4 = _align256(N * h * e), _align256(N * h * 4)
        k3 = h + 2 * m.kv_heads * m.Dh
        part = _align256(-(-N // NORM_BWD_ROWS) * h * 4)
        first = (9 * nh + 3 * nh4 + _align256(h * h * e) + _align256(m.H * N * 4) + workspace_bytes(m, WS_ATTN_BWD)
                 + part + workspace_bytes(m, WS_MLP_BWD))
        second = 2 * nh + 2 * _align256(N * k3 * e) + _align256(h * k3 * e) + nh4 + part
        return 2 * nh4 + max(first, second)
    if kind != WS_LAYER:
        raise ValueError(f"unknown workspace kind {kind}")
    total = 2 * _align256(N * h * e) + _align256(N * F * e)
    if m.rope_base > 0:
        total += _align256(N * (m.Dh // 2) * 8)
    lm = lead_rows(m)
    if lm:
        total += 7 * _align256(lm * h * 4) + _align256(lm * F * 4)
        total += _align256(_lead_part_bytes(lm, h, F, m.D, m.mlp == "swiglu"))
    return total


# ------------------------------------------------------------------- weights
def layer_weight_elems(m: Model) -> int:
    """Elements of one layer's weight matrices over all D shards: W_QKV
    [(H + 2 Hkv) Dh][h], W_O [h][h], W1 [F][h] (gated: [2F][h]), W2 [h][F],
    and the two RMSNorm gains [h]."""
    qkv = (m.H + 2 * m.kv_heads) * m.Dh * m.h
    wo = m.h * m.H * m.Dh
    w1 = (2 if m.mlp == "swiglu" else 1) * m.F * m.h
    w2 = m.h * m.F
    return qkv + wo + w1 + w2 + 2 * m.h


# --------------------------------------------------------------- rank budget
def rank_memory(m: Model, train: bool = False, save_attention: bool = False) -> dict:
    """Bytes on one rank's device at the peak of a forward over all layers
    (the layer being computed holds the transients), by component:

    weights_owned      every layer's weights / D, in dtype (paragraph 1)
    weights_received   the other D - 1 shards of the layer being computed:
                       this library applies all of a layer's attention
                       shards in one launch and keeps every MLP shard until
                       the down product, so a whole layer is present at once
    kv_local           the rank's own K and V rows of every layer (they stay
                       for the later layers' all-gathers, or for a backward)
    kv_gathered        the other ranks' K/V rows of the layer being computed
                       (transient: S - N rows, all K/V heads)
    residual           the layer's input and output rows, fp32 [N][h] each
    workspace          the layer call's scratch (WS_LAYER)

    train=True adds, for mixed-precision training with Adam (assumptions,
    the pages state none): fp32 gradients, fp32 master weights and the two
    fp32 moments of the owned weights (16 bytes per owned parameter with the
    dtype copy); each layer's fp32 input kept for its backward, which
    recomputes the rest of the layer; and the peak of one layer's backward:
    its fp32 dK/dV over the whole gathered sequence (the rank's contribution
    before the reduce-scatter that returns each row to its owner) and the
    summed rows the rank gets back, the layer backward's workspace
    (WS_LAYER_BWD), the fp32 output gradient and input gradient [N][h], and
    the fp32 weight gradients of the received shards. save_attention (with
    train) adds what tsp_layer_fwd_save keeps of each layer for
    tsp_layer_bwd_ex, so that the backward runs neither the attention
    forward nor the MLP up product again: the attention output and row
    statistics, fp32 [N][H][Dh] and [H][N], and the MLP pre-activation Z,
    [N][F] in dtype."""
    e = _elem(m.dtype)
    W = layer_weight_elems(m)
    kvw = 2 * m.kv_heads * m.Dh  # K and V elements per token
    out = {
        "weights_owned": m.layers * W * e // m.D,
        "weights_received": W * e - W * e // m.D,
        "kv_local": m.layers * m.N * kvw * e,
        "kv_gathered": (m.S - m.N) * kvw * e,
        "residual": 2 * m.N * m.h * 4,
        "workspace": workspace_bytes(m, WS_LAYER),
    }
    if train:
        out["grads_owned"] = m.layers * W * 4 // m.D
        out["optimizer_owned"] = m.layers * W * 12 // m.D
        out["saved_layer_inputs"] = m.layers * m.N * m.h * 4
        if save_attention:
            out["saved_attention"] = m.layers * (m.N * m.H * m.Dh + m.H * m.N) * 4
            out["saved_mlp_preact"] = m.layers * m.N * m.F * e
        out["backward_peak"] = ((m.S + m.N) * kvw * 4 + workspace_bytes(m, WS_LAYER_BWD) + 2 * m.N * m.h * 4
                                + (W * 4 - W * 4 // m.D))
    out["total"] = sum(out.values())
    return out


def single_gpu_bytes(m: Model, workload: str = "layer") -> int:
    """Device bytes a one-GPU run of this library allocates for its inputs,
    outputs and scratch: all D shards of every layer resident, the whole
    gathered K/V of every layer (the other ranks' rows are inputs), one fp32
    [N][h] input and its output ('layer'), or an input and two alternating
    outputs ('layers': the layer stack)."""
    e = _elem(m.dtype)
    W = layer_weight_elems(m)
    kv = m.S * 2 * m.kv_heads * m.Dh * e
    rows = m.N * m.h * 4
    n_res = 2 if workload == "layer" else 3
    return m.layers * (W * e + kv) + n_res * rows + workspace_bytes(m, WS_LAYER)


def seven_b(S: int = 131072, D: int = 8, r: int = 0, layers: int = 32, **kw) -> Model:
    """The pages' 7B dense decoder: hidden 4096, 32 heads of 128 (query and
    K/V), MLP 4x, 32 layers, bf16 (paragraph 1)."""
    return Model(S=S, D=D, r=r, h=4096, H=32, Dh=128, F=16384, layers=layers, **kw)
