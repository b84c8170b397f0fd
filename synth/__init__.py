"""Seeded synthetic inputs for the TSP rank-local layer.

This module is shared by the CPU oracle's tests and the HIP path's tests and
benchmark. It only draws random numbers, rounds them to the storage type and
names the workload shapes; it holds none of the layer's arithmetic.

Random streams: every named tensor gets its own numpy PCG64 stream keyed by
(seed, tensor id, shard, chunk). Large tensors are drawn in fixed-size chunks,
each from its own stream, so the values do not depend on the number of worker
threads used to draw them.

bf16 tensors are returned as their 16-bit patterns (numpy uint16), produced by
round-to-nearest-even from float32 draws; `bf16_to_f32` widens them exactly.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_CHUNK = 1 << 22

# Tensor ids for the per-tensor random streams.
TID_X = 1
TID_G_ATTN = 2
TID_G_MLP = 3
TID_WQKV = 10
TID_WO = 11
TID_W1 = 12
TID_W2 = 13
TID_K_REMOTE = 20
TID_V_REMOTE = 21
TID_Q = 22
TID_DY = 30  # gradient arriving at a branch output (backward tests)
TID_DK_LOC = 31  # summed K/V-row gradients handed to a layer backward's second half
TID_DV_LOC = 32


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Sizes of one decoder layer split over a folded axis of size D.

    S: total sequence, D: axis size, h: hidden, H: heads, Dh: head width,
    F: MLP width, eps: RMSNorm epsilon, dtype: 'f32' or 'bf16' storage type of
    weights and activations (accumulation is always fp32 on the device),
    Hkv: K/V heads of grouped-query attention (0 means H), mlp: 'gelu' (two
    matrices) or 'swiglu' (gated: the first matrix holds gate and up rows).
    """

    S: int
    D: int
    h: int
    H: int
    Dh: int
    F: int
    eps: float = 1e-5
    dtype: str = "bf16"
    Hkv: int = 0
    mlp: str = "gelu"

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def C(self) -> int:
        return self.S // (2 * self.D)

    @property
    def N(self) -> int:
        return self.S // self.D

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.Dh))


# Named workloads. Sizes follow the 7B dense decoder the TSP pages validate
# (hidden 4096, 32 heads of 128, MLP 4x, 128K tokens, axis of 8) and a tiny fp32
# layer for exhaustive per-rank checks.
TINY_FP32 = LayerShape(S=1024, D=4, h=256, H=4, Dh=64, F=1024, dtype="f32")
SEVEN_B = LayerShape(S=131072, D=8, h=4096, H=32, Dh=128, F=16384, dtype="bf16")

WEIGHT_STD = 0.02


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(shape, seed: int, tid: int, shard: int = 0, std: float = 1.0,
           mean: float = 0.0, dtype: str = "f32") -> np.ndarray:
    """Seeded N(mean, std^2) tensor.

    dtype 'f32' returns float32; 'bf16' returns uint16 bf16 bit patterns
    rounded from the float32 draw.
    """
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.default_rng([seed, tid, shard, i])
        seg = out[lo:hi]
        g.standard_normal(hi - lo, dtype=np.float32, out=seg)
        if std != 1.0:
            seg *= np.float32(std)
        if mean != 0.0:
            seg += np.float32(mean)

    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    out = out.reshape(shape)
    if dtype == "f32":
        return out
    if dtype == "bf16":
        return f32_to_bf16(out)
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Values of a stored tensor as float32 (bf16 widened exactly)."""
    if dtype == "bf16":
        return bf16_to_f32(a)
    return np.asarray(a, dtype=np.float32)


def layer_weights(shape: LayerShape, seed: int, gain: str = "ones") -> dict:
    """Per-shard weights of one layer, in storage type.

    Shard j of the attention projections covers query heads j*H/D ..
    (j+1)*H/D-1 and K/V heads j*Hkv/D .. (j+1)*Hkv/D-1:
      wqkv[j]: [(H + 2*Hkv)*Dh/D, h]  rows are that head group's Q rows, then
               K rows, then V rows, each head-major (head, then feature);
      wo[j]:   [h, h/D]    the W_O columns that read that head group.
    Shard j of the MLP covers hidden units j*F/D .. (j+1)*F/D-1:
      w1[j]:   [F/D, h]    rows of W1 (out, in); with mlp 'swiglu' [2F/D, h],
               the gate rows of those units, then their up rows;
      w2[j]:   [h, F/D]    columns of W2 (out, in).
    Gains g_attn, g_mlp: [h]; 'ones' or 'random' (1 + 0.1*N(0,1)).
    """
    D, h, F = shape.D, shape.h, shape.F
    hd = h // D
    hkd = shape.kv_heads * shape.Dh // D
    fd = F // D
    dt = shape.dtype
    w = {
        "wqkv": [normal((hd + 2 * hkd, h), seed, TID_WQKV, j, WEIGHT_STD, dtype=dt) for j in range(D)],
        "wo": [normal((h, hd), seed, TID_WO, j, WEIGHT_STD, dtype=dt) for j in range(D)],
        "w1": [normal(((2 if shape.mlp == "swiglu" else 1) * fd, h), seed, TID_W1, j, WEIGHT_STD, dtype=dt)
               for j in range(D)],
        "w2": [normal((h, fd), seed, TID_W2, j, WEIGHT_STD, dtype=dt) for j in range(D)],
    }
    if gain == "ones":
        one = np.ones(h, dtype=np.float32)
        w["g_attn"] = f32_to_bf16(one) if dt == "bf16" else one
        w["g_mlp"] = f32_to_bf16(one) if dt == "bf16" else one.copy()
    elif gain == "random":
        w["g_attn"] = normal((h,), seed, TID_G_ATTN, 0, 0.1, 1.0, dtype=dt)
        w["g_mlp"] = normal((h,), seed, TID_G_MLP, 0, 0.1, 1.0, dtype=dt)
    else:
        raise ValueError(gain)
    return w


def activations(rows: int, width: int, seed: int, tid: int = TID_X, dtype: str = "f32") -> np.ndarray:
    """Activations ~ N(0, 1), [rows, width]."""
    return normal((rows, width), seed, tid, 0, 1.0, dtype=dtype)


def remote_kv(shape: LayerShape, seed: int, dtype: str | None = None):
    """Full-sequence K and V, [S, Hkv, Dh], ~ N(0,1): what the all-gather would deliver."""
    dt = dtype or shape.dtype
    k = normal((shape.S, shape.kv_heads, shape.Dh), seed, TID_K_REMOTE, 0, 1.0, dtype=dt)
    v = normal((shape.S, shape.kv_heads, shape.Dh), seed, TID_V_REMOTE, 0, 1.0, dtype=dt)
    return k, v


def attn_queries(shape: LayerShape, seed: int, dtype: str | None = None) -> np.ndarray:
    """Local queries [S/D, H, Dh] ~ N(0,1)."""
    dt = dtype or shape.dtype
    return normal((shape.N, shape.H, shape.Dh), seed, TID_Q, 0, 1.0, dtype=dt)
