"""Host-only checks of the C ABI: the library loads, exports what include/tsp.h
declares, the host zigzag map matches the oracle bit for bit, and every
argument error is reported before anything is enqueued (no GPU needed: none
of these calls reaches a launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import tsp_rank_local_amd as tsp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "tsp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsp_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = tsp.lib()
    declared = _header_functions()
    assert declared == sorted(tsp.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.tsp_abi_version() == 3


def test_status_strings():
    L = tsp.lib()
    assert L.tsp_status_string(0) == b"ok"
    assert L.tsp_status_string(3) == b"workspace too small"
    assert L.tsp_status_string(99) == b"unknown status"


@pytest.mark.parametrize("S,D", [(16, 4), (1024, 4), (64, 1), (96, 3), (131072, 8), (2400, 4)])
def test_zigzag_host_matches_oracle(S, D):
    for r in range(D):
        got = tsp.tsp_zigzag_index_host(S, D, r)
        assert got.dtype == np.int32
        assert np.array_equal(got.astype(np.int64), oracle.zigzag_positions(S, D, r))


def _shape(**kw):
    base = dict(S=1024, D=4, r=0, h=256, H=4, Dh=64, F=1024, eps=1e-5, scale=0.125, dtype="f32")
    base.update(kw)
    return tsp.make_shape(**base)


def _a256(n):
    return (n + 255) // 256 * 256


def _lead_bytes(S, D, h, F, gated=False):
    """bf16 rank 0 also recomputes its first m = min(64, S/(2D)) rows in fp32:
    seven [m][h] and one [m][F] fp32 buffers, plus the K-chunk partial sums of
    the largest of its four products (chunk: 512, 256, 128 or 64 dividing the
    reduction segment; a gated MLP up has 2F product columns)."""
    m = min(64, S // (2 * D))
    hd, fd = h // D, F // D
    chunk = lambda k: next(c for c in (512, 256, 128, 64) if k % c == 0)
    up = h // chunk(h) * m * (2 * F if gated else F)
    part = 4 * max(h // chunk(h) * m * 3 * h, h // chunk(hd) * m * h, up, F // chunk(fd) * m * h)
    return 7 * _a256(m * h * 4) + _a256(m * F * 4) + _a256(part)


def test_workspace_sizes():
    # MLP: GELU(x W1_j^T) of every ring step side by side, [N][F] in the dtype;
    # layer: Q (later RMSNorm(h1)) and RMSNorm(x) (later O), [N][h] each, plus that
    N, h, F = 256, 256, 1024
    for r in (0, 1):
        s = _shape(dtype="bf16", r=r)
        assert tsp.workspace_size(s, tsp.TSP_WS_MLP) == N * F * 2
        lead = _lead_bytes(1024, 4, h, F) if r == 0 else 0
        assert tsp.workspace_size(s, tsp.TSP_WS_LAYER) == 2 * N * h * 2 + N * F * 2 + lead
    s = _shape(dtype="f32")
    assert tsp.workspace_size(s, tsp.TSP_WS_LAYER) == 2 * N * h * 4 + N * F * 4
    for r in (0, 3):
        s7 = tsp.make_shape(131072, 8, r, 4096, 32, 128, 16384, dtype="bf16")
        lead = _lead_bytes(131072, 8, 4096, 16384) if r == 0 else 0
        assert tsp.workspace_size(s7, tsp.TSP_WS_LAYER) == 2 * 16384 * 4096 * 2 + 16384 * 16384 * 2 + lead
    # gated MLP: the hidden layer is still [N][F]; only the leading rows'
    # partial sums of the up product double
    s7g = tsp.make_shape(131072, 8, 0, 4096, 32, 128, 16384, dtype="bf16", mlp="swiglu")
    assert tsp.workspace_size(s7g, tsp.TSP_WS_MLP) == 16384 * 16384 * 2
    assert tsp.workspace_size(s7g, tsp.TSP_WS_LAYER) == (2 * 16384 * 4096 * 2 + 16384 * 16384 * 2 +
                                                         _lead_bytes(131072, 8, 4096, 16384, gated=True))


def test_grouped_kv_shapes_accepted():
    """Grouped K/V heads change no workspace buffer (Q, O and the MLP input
    keep H heads); Hkv = H is the same as Hkv = 0."""
    base = tsp.workspace_size(_shape(dtype="bf16", H=8, h=512), tsp.TSP_WS_LAYER)
    for hkv in (0, 4, 8):
        assert tsp.workspace_size(_shape(dtype="bf16", H=8, h=512, Hkv=hkv), tsp.TSP_WS_LAYER) == base
    # rotation with whole 128-column Q and K blocks per shard
    tsp.workspace_size(_shape(dtype="bf16", H=8, h=512, Hkv=4, D=2, rope_base=1e4), tsp.TSP_WS_LAYER)


@pytest.mark.parametrize("kw,code", [
    (dict(S=1020), tsp.TSP_ERR_INVALID_ARG),          # S not a multiple of 2D
    (dict(S=0), tsp.TSP_ERR_INVALID_ARG),             # empty sequence
    (dict(S=1 << 31), tsp.TSP_ERR_INVALID_ARG),       # positions must fit int32
    (dict(r=4), tsp.TSP_ERR_INVALID_ARG),             # r out of range
    (dict(D=0), tsp.TSP_ERR_INVALID_ARG),
    (dict(D=65, S=130), tsp.TSP_ERR_INVALID_ARG),     # D above the limit
    (dict(Dh=32, h=128), tsp.TSP_ERR_UNSUPPORTED),
    (dict(h=512), tsp.TSP_ERR_INVALID_ARG),           # h != H*Dh
    (dict(H=3, h=192), tsp.TSP_ERR_INVALID_ARG),      # H % D
    (dict(F=1002), tsp.TSP_ERR_INVALID_ARG),          # F % D
    (dict(F=4 * 96), tsp.TSP_ERR_UNSUPPORTED),        # F/D not a multiple of 64
    (dict(dtype=7), tsp.TSP_ERR_INVALID_ARG),
    (dict(eps=-1.0), tsp.TSP_ERR_INVALID_ARG),
    (dict(scale=float("nan")), tsp.TSP_ERR_INVALID_ARG),
    (dict(rope_base=-1.0), tsp.TSP_ERR_INVALID_ARG),
    (dict(rope_base=float("inf")), tsp.TSP_ERR_INVALID_ARG),
    (dict(rope_base=1e4, dtype="bf16"), tsp.TSP_ERR_UNSUPPORTED),  # h/D = 64: rotation needs whole 128-column heads
    (dict(mlp=2), tsp.TSP_ERR_INVALID_ARG),           # unknown MLP kind
    (dict(mlp=-1), tsp.TSP_ERR_INVALID_ARG),
    (dict(Hkv=-1), tsp.TSP_ERR_INVALID_ARG),
    (dict(Hkv=3), tsp.TSP_ERR_INVALID_ARG),           # Hkv must divide H
    (dict(Hkv=8), tsp.TSP_ERR_INVALID_ARG),           # more K/V heads than query heads
    (dict(Hkv=2), tsp.TSP_ERR_INVALID_ARG),           # Hkv % D: a head group needs whole K/V heads
    (dict(H=8, h=512, Hkv=4, rope_base=1e4, dtype="bf16"),
     tsp.TSP_ERR_UNSUPPORTED),                        # h/D = 128 but Hkv*Dh/D = 64: no whole 128-column K block
])
def test_shape_errors(kw, code):
    with pytest.raises(tsp.TspError) as ei:
        tsp.workspace_size(_shape(**kw), tsp.TSP_WS_LAYER)
    assert ei.value.status == code
    assert tsp.lib().tsp_last_error()  # a message explains it


FAKE = 1 << 40  # a 16-byte aligned address that is never dereferenced


def test_pointer_errors_enqueue_nothing():
    s = _shape()
    # null / misaligned pointers on attention
    for q, code in [(None, tsp.TSP_ERR_INVALID_ARG), (FAKE + 4, tsp.TSP_ERR_INVALID_ARG)]:
        with pytest.raises(tsp.TspError) as ei:
            tsp.tsp_zigzag_attn(s, q, FAKE, FAKE + (1 << 30), FAKE + (2 << 30), stream=0)
        assert ei.value.status == code
    # output overlapping an input
    with pytest.raises(tsp.TspError) as ei:
        tsp.tsp_zigzag_attn(s, FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (1 << 30) + 4096, stream=0)
    assert ei.value.status == tsp.TSP_ERR_INVALID_ARG and b"overlap" in tsp.lib().tsp_last_error()
    # grouped K/V heads: k and v hold S*Hkv*Dh elements; an o over the last
    # bytes of a 1-head k overlaps it
    s1 = _shape(Hkv=1)
    kv1 = 1024 * 1 * 64 * 4
    with pytest.raises(tsp.TspError) as ei:
        tsp.tsp_zigzag_attn(s1, FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (1 << 30) + kv1 - 256, stream=0)
    assert b"overlap" in tsp.lib().tsp_last_error()
    # fp32 inputs with a bf16 output
    with pytest.raises(tsp.TspError):
        tsp.tsp_zigzag_attn(s, FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), tsp.TSP_BF16, stream=0)
    # flags: unknown bits; pre-scaled Q needs bf16 q and o
    sb = _shape(dtype="bf16")
    args = (FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30))
    for shape, odt, flags, code in [(sb, tsp.TSP_BF16, 2, tsp.TSP_ERR_INVALID_ARG),
                                    (s, tsp.TSP_F32, tsp.TSP_ATTN_Q_LOG2_SCALED, tsp.TSP_ERR_UNSUPPORTED),
                                    (sb, tsp.TSP_F32, tsp.TSP_ATTN_Q_LOG2_SCALED, tsp.TSP_ERR_UNSUPPORTED)]:
        with pytest.raises(tsp.TspError) as ei:
            tsp.tsp_zigzag_attn_ex(shape, *args, odt, flags, stream=0)
        assert ei.value.status == code


def test_mlp_errors():
    s = _shape()
    w = [FAKE + (i << 24) for i in range(4)]
    need = tsp.workspace_size(s, tsp.TSP_WS_MLP)
    with pytest.raises(tsp.TspError) as ei:  # workspace too small
        tsp.tsp_mlp_ring(s, FAKE + (1 << 32), w, w, None, FAKE + (2 << 32), FAKE + (3 << 32), need - 1, stream=0)
    assert ei.value.status == tsp.TSP_ERR_WORKSPACE
    bad = list(w)
    bad[2] = None
    with pytest.raises(tsp.TspError) as ei:  # a null shard pointer
        tsp.tsp_mlp_ring(s, FAKE + (1 << 32), w, bad, None, FAKE + (2 << 32), FAKE + (3 << 32), need, stream=0)
    assert ei.value.status == tsp.TSP_ERR_INVALID_ARG and b"w2[2]" in tsp.lib().tsp_last_error()
    with pytest.raises(tsp.TspError):  # x overlaps y
        tsp.tsp_mlp_ring(s, FAKE, w, w, None, FAKE + 256, FAKE + (3 << 32), need, stream=0)


def test_mlp_bwd_workspace_and_errors():
    # W1 stacked, W1^T, W2^T ([F][h] each), x^T and dy^T ([h][N]), Z^T and
    # GELU(Z)^T ([F][N]), all in the dtype
    for dtype, e in (("f32", 4), ("bf16", 2)):
        s = _shape(dtype=dtype)
        N, h, F = 256, 256, 1024
        assert tsp.workspace_size(s, tsp.TSP_WS_MLP_BWD) == (3 * F * h + 2 * h * N + 2 * F * N) * e
    s7 = tsp.make_shape(131072, 8, 3, 4096, 32, 128, 16384, dtype="bf16")
    assert tsp.workspace_size(s7, tsp.TSP_WS_MLP_BWD) == (3 * 16384 * 4096 + 2 * 4096 * 16384 + 2 * 16384 ** 2) * 2
    s = _shape(dtype="bf16")
    need = tsp.workspace_size(s, tsp.TSP_WS_MLP_BWD)
    w = [FAKE + (i << 24) for i in range(4)]
    g = [FAKE + (1 << 36) + (i << 24) for i in range(4)]
    x, dy, dx, ws = FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32), FAKE + (4 << 32)

    def call(shape=s, x=x, dy=dy, dx=dx, dw1=g, dw2=g, ws=ws, nbytes=need, res=None):
        with pytest.raises(tsp.TspError) as ei:
            tsp.tsp_mlp_ring_bwd(shape, x, w, w, dy, res, dx, dw1, dw2, ws, nbytes, stream=0)
        return ei.value.status, tsp.lib().tsp_last_error()

    assert call(nbytes=need - 1)[0] == tsp.TSP_ERR_WORKSPACE
    bad = list(g)
    bad[1] = None
    st, msg = call(dw2=bad)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"dw2[1]" in msg
    assert call(dx=x + 512)[0] == tsp.TSP_ERR_INVALID_ARG                       # dx overlaps x
    assert call(dw1=[ws + 256] + g[1:])[0] == tsp.TSP_ERR_INVALID_ARG           # dW1 inside the workspace
    assert call(res=dx + 64)[0] == tsp.TSP_ERR_INVALID_ARG                      # residual partly over dx
    assert call(dy=dy + 8)[0] == tsp.TSP_ERR_INVALID_ARG                        # misaligned
    assert call(shape=_shape(dtype="bf16", mlp="swiglu"))[0] == tsp.TSP_ERR_UNSUPPORTED
    # S/D = 96 tokens: not a multiple of 64 (K of the weight-gradient products)
    st = call(shape=tsp.make_shape(384, 4, 0, 256, 4, 64, 1024, dtype="bf16"), nbytes=1 << 40)[0]
    assert st == tsp.TSP_ERR_UNSUPPORTED
    # S/D = 4194304 tokens: past the 65535 x 64 rows of a layout pass and the
    # 32-bit offsets of the token-K products; rejected before anything runs
    # (the stream argument 0 would be the default stream: nothing may reach it)
    st, msg = call(shape=tsp.make_shape(2 * 4194304, 2, 0, 64, 1, 64, 128, dtype="bf16"), nbytes=1 << 60)
    assert st == tsp.TSP_ERR_UNSUPPORTED and b"S/D" in msg
    with pytest.raises(tsp.TspError):
        tsp.workspace_size(tsp.make_shape(2 * 4194304, 2, 0, 64, 1, 64, 128, dtype="bf16"), tsp.TSP_WS_MLP_BWD)
    with pytest.raises(tsp.TspError):
        tsp.workspace_size(_shape(dtype="bf16", mlp="swiglu"), tsp.TSP_WS_MLP_BWD)


def test_attn_bwd_workspace_and_errors():
    # log-sum-exp and Delta of every (head, local row), fp32
    s = _shape(dtype="bf16")
    assert tsp.workspace_size(s, tsp.TSP_WS_ATTN_BWD) == 2 * 4 * 256 * 4
    s7 = tsp.make_shape(131072, 8, 0, 4096, 32, 128, 16384, dtype="bf16")
    assert tsp.workspace_size(s7, tsp.TSP_WS_ATTN_BWD) == 2 * 32 * 16384 * 4
    need = tsp.workspace_size(s, tsp.TSP_WS_ATTN_BWD)
    q, k, v, do = (FAKE + (i << 32) for i in range(4))
    dq, dk, dv, ws = (FAKE + ((5 + i) << 32) for i in range(4))

    def call(shape=s, nbytes=need, **kw):
        a = dict(q=q, k=k, v=v, do=do, dq=dq, dk=dk, dv=dv, ws=ws)
        a.update(kw)
        with pytest.raises(tsp.TspError) as ei:
            tsp.tsp_zigzag_attn_bwd(shape, a["q"], a["k"], a["v"], a["do"], a["dq"], a["dk"], a["dv"],
                                    a["ws"], nbytes, stream=0)
        return ei.value.status, tsp.lib().tsp_last_error()

    assert call(nbytes=need - 1)[0] == tsp.TSP_ERR_WORKSPACE
    st, msg = call(do=None)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"dout is NULL" in msg
    st, msg = call(dk=k + 4096)  # an output over an input
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlap" in msg
    st, msg = call(dv=dk + 256)  # two outputs over each other
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlap" in msg
    assert call(dq=dq + 4)[0] == tsp.TSP_ERR_INVALID_ARG
    assert call(shape=_shape(dtype="bf16", Dh=32, H=8))[0] == tsp.TSP_ERR_UNSUPPORTED


def test_attn_bwd_ex_errors():
    s = _shape(dtype="bf16")
    need = tsp.workspace_size(s, tsp.TSP_WS_ATTN_BWD)
    q, k, v, do = (FAKE + (i << 32) for i in range(4))
    dq, dk, dv, ws, o, lse = (FAKE + ((5 + i) << 32) for i in range(6))

    def call(shape=s, o=None, lse=None, flags=tsp.TSP_ATTN_BWD_PLAIN_PDS):
        with pytest.raises(tsp.TspError) as ei:
            tsp.tsp_zigzag_attn_bwd_ex(shape, q, k, v, o, lse, do, dq, dk, dv, flags, ws, need - 1, stream=0)
        return ei.value.status, tsp.lib().tsp_last_error()

    assert call()[0] == tsp.TSP_ERR_WORKSPACE  # everything else valid
    st, msg = call(flags=2)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"flags" in msg
    st, msg = call(o=o)  # o without lse
    assert st == tsp.TSP_ERR_INVALID_ARG and b"lse is NULL" in msg
    assert call(o=o, lse=lse)[0] == tsp.TSP_ERR_WORKSPACE
    assert call(shape=_shape())[0] == tsp.TSP_ERR_UNSUPPORTED  # plain P and dS in fp32


def test_attn_bwd_noalloc_errors():
    """The entry point without a workspace checks every argument, and the size
    of its static scratch, before it looks the scratch up or enqueues
    anything (so these run without a GPU)."""
    s = _shape(dtype="bf16")
    q, k, v, do = (FAKE + (i << 32) for i in range(4))
    dq, dk, dv = (FAKE + ((5 + i) << 32) for i in range(3))

    def call(shape=s, **kw):
        a = dict(q=q, k=k, v=v, do=do, dq=dq, dk=dk, dv=dv)
        a.update(kw)
        with pytest.raises(tsp.TspError) as ei:
            tsp.tsp_zigzag_attn_bwd_noalloc(shape, a["q"], a["k"], a["v"], a["do"], a["dq"], a["dk"], a["dv"],
                                            stream=0)
        return ei.value.status, tsp.lib().tsp_last_error()

    st, msg = call(do=None)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"dout is NULL" in msg
    st, msg = call(dk=k + 4096)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlap" in msg
    # H * S/D above 1048576 statistics: the 8 MiB array cannot hold them
    big = tsp.make_shape(524288, 8, 0, 4096, 32, 128, 16384, dtype="bf16")
    st, msg = call(shape=big, q=FAKE, k=FAKE + (1 << 40), v=FAKE + (2 << 40), do=FAKE + (3 << 40),
                   dq=FAKE + (4 << 40), dk=FAKE + (5 << 40), dv=FAKE + (6 << 40))
    assert st == tsp.TSP_ERR_UNSUPPORTED and b"static" in msg
    assert call(shape=_shape(dtype="bf16", Dh=32, H=8))[0] == tsp.TSP_ERR_UNSUPPORTED


def test_attn_lse_entry_points_errors():
    sb, sf = _shape(dtype="bf16"), _shape(dtype="f32")
    q, k, v, o, lse, do = (FAKE + (i << 32) for i in range(6))
    dq, dk, dv, ws = (FAKE + ((7 + i) << 32) for i in range(4))
    need = tsp.workspace_size(sb, tsp.TSP_WS_ATTN_BWD)
    with pytest.raises(tsp.TspError) as ei:  # bf16 inputs only
        tsp.tsp_zigzag_attn_lse(sf, q, k, v, o, lse, stream=0)
    assert ei.value.status == tsp.TSP_ERR_UNSUPPORTED
    with pytest.raises(tsp.TspError) as ei:  # lse over o
        tsp.tsp_zigzag_attn_lse(sb, q, k, v, o, o + 256, stream=0)
    assert ei.value.status == tsp.TSP_ERR_INVALID_ARG and b"overlap" in tsp.lib().tsp_last_error()
    with pytest.raises(tsp.TspError) as ei:  # the statistics are required
        tsp.tsp_zigzag_attn_bwd_lse(sb, q, k, v, o, None, do, dq, dk, dv, ws, need, stream=0)
    assert ei.value.status == tsp.TSP_ERR_INVALID_ARG and b"lse is NULL" in tsp.lib().tsp_last_error()
    with pytest.raises(tsp.TspError) as ei:
        tsp.tsp_zigzag_attn_bwd_lse(sf, q, k, v, o, lse, do, dq, dk, dv, ws, need, stream=0)
    assert ei.value.status == tsp.TSP_ERR_UNSUPPORTED
    with pytest.raises(tsp.TspError) as ei:  # dq over the given o
        tsp.tsp_zigzag_attn_bwd_lse(sb, q, k, v, o, lse, do, o + 4096, dk, dv, ws, need, stream=0)
    assert ei.value.status == tsp.TSP_ERR_INVALID_ARG and b"overlap" in tsp.lib().tsp_last_error()


def test_mlp_z_entry_points_errors():
    sb, sf = _shape(dtype="bf16"), _shape(dtype="f32")
    w = [FAKE + (i << 24) for i in range(4)]
    g = [FAKE + (1 << 36) + (i << 24) for i in range(4)]
    x, y, z, ws, dy, dx = (FAKE + (i << 32) for i in range(1, 7))
    need = tsp.workspace_size(sb, tsp.TSP_WS_MLP)
    with pytest.raises(tsp.TspError) as ei:  # bf16 only
        tsp.tsp_mlp_ring_z(sf, x, w, w, None, y, z, ws, need, stream=0)
    assert ei.value.status == tsp.TSP_ERR_UNSUPPORTED
    with pytest.raises(tsp.TspError) as ei:  # z over y
        tsp.tsp_mlp_ring_z(sb, x, w, w, None, y, y + 256, ws, need, stream=0)
    assert ei.value.status == tsp.TSP_ERR_INVALID_ARG and b"z overlaps" in tsp.lib().tsp_last_error()
    with pytest.raises(tsp.TspError) as ei:
        tsp.tsp_mlp_ring_z(sb, x, w, w, None, y, None, ws, need, stream=0)
    assert ei.value.status == tsp.TSP_ERR_INVALID_ARG and b"z is NULL" in tsp.lib().tsp_last_error()
    nb = tsp.workspace_size(sb, tsp.TSP_WS_MLP_BWD)
    with pytest.raises(tsp.TspError) as ei:
        tsp.tsp_mlp_ring_bwd_z(sf, x, z, w, w, dy, None, dx, g, g, ws, nb, stream=0)
    assert ei.value.status == tsp.TSP_ERR_UNSUPPORTED
    with pytest.raises(tsp.TspError) as ei:  # z inside the workspace
        tsp.tsp_mlp_ring_bwd_z(sb, x, ws + 1024, w, w, dy, None, dx, g, g, ws, nb, stream=0)
    assert ei.value.status == tsp.TSP_ERR_INVALID_ARG and b"z overlaps" in tsp.lib().tsp_last_error()


def test_layer_errors():
    s = _shape()
    w = dict(g_attn=FAKE, g_mlp=FAKE, wqkv=[FAKE] * 4, wo=[FAKE] * 4, w1=[FAKE] * 4, w2=[FAKE] * 4)
    need = tsp.workspace_size(s, tsp.TSP_WS_LAYER)
    args = dict(x=FAKE + (1 << 32), k_full=FAKE + (2 << 32), v_full=FAKE + (3 << 32), y=FAKE + (4 << 32),
                ws=FAKE + (5 << 32))
    for phases in (0, 4, 7):
        with pytest.raises(tsp.TspError):
            tsp.tsp_layer_fwd(s, w, args["x"], args["k_full"], args["v_full"], args["y"], phases, args["ws"], need, stream=0)
    with pytest.raises(tsp.TspError) as ei:
        tsp.tsp_layer_fwd(s, w, args["x"], args["k_full"], args["v_full"], args["y"], 3, args["ws"], need - 256, stream=0)
    assert ei.value.status == tsp.TSP_ERR_WORKSPACE
    with pytest.raises(tsp.TspError) as ei:  # y aliases x
        tsp.tsp_layer_fwd(s, w, args["x"], args["k_full"], args["v_full"], args["x"], 3, args["ws"], need, stream=0)
    assert b"overlaps" in tsp.lib().tsp_last_error()
    w_bad = dict(w, wo=[FAKE, FAKE, FAKE + 8, FAKE])
    with pytest.raises(tsp.TspError) as ei:
        tsp.tsp_layer_fwd(s, w_bad, args["x"], args["k_full"], args["v_full"], args["y"], 3, args["ws"], need, stream=0)
    assert b"wo[2]" in tsp.lib().tsp_last_error()


def test_zigzag_index_errors():
    with pytest.raises(tsp.TspError):
        tsp.tsp_zigzag_index_host(10, 4, 0)
    with pytest.raises(tsp.TspError):
        tsp.tsp_zigzag_index(16, 4, 0, None, stream=0)
    pos = (ctypes.c_int32 * 4)()
    assert tsp.lib().tsp_zigzag_index_host(16, 4, 1, pos) == 0
    assert list(pos) == [2, 3, 12, 13]


def test_layer_fwd_save_errors():
    """The training forward checks o_save and lse_save like every other
    argument and needs bf16; nothing is enqueued on any error."""
    w = dict(g_attn=FAKE, g_mlp=FAKE, wqkv=[FAKE] * 4, wo=[FAKE] * 4, w1=[FAKE] * 4, w2=[FAKE] * 4)
    a = dict(x=FAKE + (1 << 32), k_full=FAKE + (2 << 32), v_full=FAKE + (3 << 32), y=FAKE + (4 << 32),
             ws=FAKE + (5 << 32), o=FAKE + (6 << 32), lse=FAKE + (7 << 32), z=None)

    def call(shape=None, **kw):
        s = shape or _shape(dtype="bf16")
        b = dict(a)
        b.update(kw)
        with pytest.raises(tsp.TspError) as ei:
            tsp.tsp_layer_fwd_save(s, w, b["x"], b["k_full"], b["v_full"], b["y"], b["o"], b["lse"], 3, b["ws"],
                                   tsp.workspace_size(s, tsp.TSP_WS_LAYER), stream=0, z_save=b["z"])
        return ei.value.status, tsp.lib().tsp_last_error()

    st, msg = call(o=None)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"o_save is NULL" in msg
    st, msg = call(lse=None)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"lse_save is NULL" in msg
    assert call(shape=_shape(dtype="f32"))[0] == tsp.TSP_ERR_UNSUPPORTED
    st, msg = call(o=a["y"] + 1024)  # O over y
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg
    st, msg = call(lse=a["ws"] + 4096)  # statistics inside the workspace
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg
    assert call(o=a["o"] + 8)[0] == tsp.TSP_ERR_INVALID_ARG  # misaligned
    # the kept MLP pre-activation: GELU MLP only, checked like the rest
    z = FAKE + (8 << 32)
    assert call(shape=_shape(dtype="bf16", mlp="swiglu"), z=z)[0] == tsp.TSP_ERR_UNSUPPORTED
    st, msg = call(z=a["y"] + 4096)  # Z over y
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg
    assert call(z=z + 8)[0] == tsp.TSP_ERR_INVALID_ARG  # misaligned


def test_layer_bwd_ex_errors():
    """tsp_layer_bwd_ex: the saved O and statistics come together, need bf16
    and must not overlap an output; nothing is enqueued on any error."""
    s = _shape(dtype="bf16")
    need = tsp.workspace_size(s, tsp.TSP_WS_LAYER_BWD)
    w = dict(g_attn=FAKE, g_mlp=FAKE, wqkv=[FAKE] * 4, wo=[FAKE] * 4, w1=[FAKE] * 4, w2=[FAKE] * 4)

    def gl(base):
        return [FAKE + (base << 32) + (i << 28) for i in range(4)]

    grads = dict(g_attn=FAKE + (20 << 32), g_mlp=FAKE + (21 << 32), wqkv=gl(22), wo=gl(23), w1=gl(24), w2=gl(25))
    a = dict(x=FAKE + (1 << 32), k_full=FAKE + (2 << 32), v_full=FAKE + (3 << 32), dy=FAKE + (4 << 32),
             dk_full=FAKE + (5 << 32), dv_full=FAKE + (6 << 32), dk_loc=FAKE + (7 << 32), dv_loc=FAKE + (8 << 32),
             dx=FAKE + (9 << 32), ws=FAKE + (10 << 32), o=FAKE + (11 << 32), lse=FAKE + (12 << 32), z=None)

    def call(shape=s, **kw):
        b = dict(a)
        b.update(kw)
        with pytest.raises(tsp.TspError) as ei:
            tsp.tsp_layer_bwd_ex(shape, w, b["x"], b["k_full"], b["v_full"], b["dy"], b["o"], b["lse"], b["dk_full"],
                                 b["dv_full"], b["dk_loc"], b["dv_loc"], b["dx"], grads, tsp.TSP_BWD_ATTN, b["ws"],
                                 need if shape is s else 1 << 40, stream=0, z_saved=b["z"])
        return ei.value.status, tsp.lib().tsp_last_error()

    st, msg = call(lse=None)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"both" in msg
    st, msg = call(o=None)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"both" in msg
    assert call(shape=_shape(dtype="f32"))[0] == tsp.TSP_ERR_UNSUPPORTED
    st, msg = call(dk_full=a["o"] + 4096)  # an output over the saved O
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg
    st, msg = call(o=a["ws"])  # the saved O inside the workspace
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg
    assert call(lse=a["lse"] + 8)[0] == tsp.TSP_ERR_INVALID_ARG  # misaligned
    st, msg = call(o=None, lse=None, z=FAKE + (13 << 32))  # Z alone
    assert st == tsp.TSP_ERR_INVALID_ARG and b"z_saved needs" in msg
    st, msg = call(z=a["dk_full"])  # Z over an output
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg


def test_layer_bwd_workspace_and_errors():
    # dh1, dq fp32 [N][h]; then the larger phase: nine [N][h] in dtype, three
    # fp32 [N][h], W_O^T, the forward's lse [H][N], the attention backward's
    # statistics, the gain partials and the MLP backward's scratch; or xn, xn^T,
    # [dq|dk|dv] and its transpose, W_QKV^T, dxn, the gain partials
    for dtype, e in (("f32", 4), ("bf16", 2)):
        s = _shape(dtype=dtype)
        N, h, H, F, k3 = 256, 256, 4, 1024, 3 * 256
        part = (N // 16) * h * 4
        mlp = (3 * F * h + 2 * h * N + 2 * F * N) * e
        first = 9 * N * h * e + 3 * N * h * 4 + h * h * e + H * N * 4 + 2 * H * N * 4 + part + mlp
        second = 2 * N * h * e + 2 * N * k3 * e + h * k3 * e + N * h * 4 + part
        assert tsp.workspace_size(s, tsp.TSP_WS_LAYER_BWD) == 2 * N * h * 4 + max(first, second)
    s = _shape(dtype="bf16")
    need = tsp.workspace_size(s, tsp.TSP_WS_LAYER_BWD)
    w = dict(g_attn=FAKE, g_mlp=FAKE, wqkv=[FAKE] * 4, wo=[FAKE] * 4, w1=[FAKE] * 4, w2=[FAKE] * 4)

    def gl(base):
        return [FAKE + (base << 32) + (i << 28) for i in range(4)]

    grads = dict(g_attn=FAKE + (20 << 32), g_mlp=FAKE + (21 << 32), wqkv=gl(22), wo=gl(23), w1=gl(24), w2=gl(25))
    a = dict(x=FAKE + (1 << 32), k_full=FAKE + (2 << 32), v_full=FAKE + (3 << 32), dy=FAKE + (4 << 32),
             dk_full=FAKE + (5 << 32), dv_full=FAKE + (6 << 32), dk_loc=FAKE + (7 << 32), dv_loc=FAKE + (8 << 32),
             dx=FAKE + (9 << 32), ws=FAKE + (10 << 32))

    def call(shape=s, phases=tsp.TSP_BWD_ATTN, nbytes=need, g=grads, wt=w, **kw):
        b = dict(a)
        b.update(kw)
        with pytest.raises(tsp.TspError) as ei:
            tsp.tsp_layer_bwd(shape, wt, b["x"], b["k_full"], b["v_full"], b["dy"], b["dk_full"], b["dv_full"],
                              b["dk_loc"], b["dv_loc"], b["dx"], g, phases, b["ws"], nbytes, stream=0)
        return ei.value.status, tsp.lib().tsp_last_error()

    for phases in (0, 4, 7):
        assert call(phases=phases)[0] == tsp.TSP_ERR_INVALID_ARG
    st, msg = call(phases=tsp.TSP_BWD_ALL)  # both halves in one call: D = 1 only
    assert st == tsp.TSP_ERR_INVALID_ARG and b"D=1" in msg
    assert call(nbytes=need - 1)[0] == tsp.TSP_ERR_WORKSPACE
    st, msg = call(dy=None)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"dy is NULL" in msg
    st, msg = call(g=dict(grads, wo=grads["wo"][:2] + [None] + grads["wo"][3:]))
    assert st == tsp.TSP_ERR_INVALID_ARG and b"grads->wo[2]" in msg
    # a phase checks only what it uses: the QKV half needs no dy, no K/V and
    # no MLP gradients, but its own dk_loc and dx
    st, msg = call(phases=tsp.TSP_BWD_QKV, dy=None, k_full=None, g=dict(grads, w1=None, g_mlp=None), dk_loc=None)
    assert st == tsp.TSP_ERR_INVALID_ARG and b"dk_loc is NULL" in msg
    st, msg = call(phases=tsp.TSP_BWD_QKV, dx=a["x"] + 1024)  # dx over x
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg
    st, msg = call(dv_full=a["dk_full"] + 4096)  # two outputs over each other
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg
    st, msg = call(g=dict(grads, w2=[a["ws"] + 256] + grads["w2"][1:]))  # a gradient inside the workspace
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg
    st, msg = call(g=dict(grads, g_mlp=a["v_full"]))  # a gradient over an input
    assert st == tsp.TSP_ERR_INVALID_ARG and b"overlaps" in msg
    assert call(dk_full=a["dk_full"] + 8)[0] == tsp.TSP_ERR_INVALID_ARG  # misaligned
    # what the backward does not cover
    assert call(shape=_shape(dtype="bf16", mlp="swiglu"), nbytes=1 << 40)[0] == tsp.TSP_ERR_UNSUPPORTED
    assert call(shape=_shape(dtype="bf16", rope_base=1e4), nbytes=1 << 40)[0] == tsp.TSP_ERR_UNSUPPORTED
    st = call(shape=tsp.make_shape(384, 4, 0, 256, 4, 64, 1024, dtype="bf16"), nbytes=1 << 40)[0]
    assert st == tsp.TSP_ERR_UNSUPPORTED  # S/D = 96
    st, msg = call(shape=tsp.make_shape(1024, 1, 0, 8320, 65, 128, 1024, dtype="bf16"), nbytes=1 << 40)
    assert st == tsp.TSP_ERR_UNSUPPORTED and b"h=8320" in msg
    for bad in (_shape(dtype="bf16", mlp="swiglu"), _shape(dtype="bf16", rope_base=1e4)):
        with pytest.raises(tsp.TspError):
            tsp.workspace_size(bad, tsp.TSP_WS_LAYER_BWD)
    # 7B: a few GB of scratch for one rank's layer backward
    s7 = tsp.make_shape(131072, 8, 0, 4096, 32, 128, 16384, dtype="bf16")
    assert 3e9 < tsp.workspace_size(s7, tsp.TSP_WS_LAYER_BWD) < 5e9
