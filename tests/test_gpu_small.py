"""GPU parity at sizes the oracle finishes in seconds: every entry point of the
C ABI against the fp64 oracle on the same seeded inputs, including ragged
tiles (chunks that are not a multiple of the tile), D = 1, the smallest
sequence, every rank, both dtypes and both K/V modes of the layer."""
import numpy as np
import pytest

import oracle
import synth
import tsp_rank_local_amd as tsp
from gpu_util import TOL_BF16, TOL_F32, assert_close, down, f64, log, torch_cuda, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_cuda()
    tsp.lib()
    return t


def _sync(torch):
    torch.cuda.synchronize()


# ---------------------------------------------------------------- zigzag
@pytest.mark.parametrize("S,D", [(16, 4), (1024, 4), (2400, 4), (131072, 8), (64, 1), (8, 4)])
def test_zigzag_index_bit_exact(torch, S, D):
    for r in range(D):
        pos = torch.full((S // D,), -1, dtype=torch.int32, device="cuda")
        tsp.tsp_zigzag_index(S, D, r, pos)
        _sync(torch)
        assert np.array_equal(pos.cpu().numpy().astype(np.int64), oracle.zigzag_positions(S, D, r))


# ---------------------------------------------------------------- attention
ATTN_CASES = [
    # S, D, H, Dh, dtype, o_dtype
    (1024, 4, 4, 64, "f32", "f32"),     # the tiny fp32 layer's attention
    (1024, 4, 2, 128, "f32", "f32"),
    (2048, 2, 2, 128, "bf16", "f32"),
    (1200, 4, 2, 128, "bf16", "f32"),   # C = 150: ragged query and key tiles
    (600, 3, 3, 64, "bf16", "f32"),     # C = 100, D = 3
    (512, 1, 3, 64, "bf16", "f32"),     # D = 1: plain causal attention
    (4096, 4, 2, 128, "bf16", "bf16"),
    (2048, 4, 4, 64, "bf16", "bf16"),
    (8, 4, 1, 64, "bf16", "f32"),       # one token per chunk
]


@pytest.mark.parametrize("S,D,H,Dh,dtype,odt", ATTN_CASES)
def test_zigzag_attention(torch, S, D, H, Dh, dtype, odt):
    shape = synth.LayerShape(S=S, D=D, h=H * Dh, H=H, Dh=Dh, F=64 * D, dtype=dtype)
    k, v = synth.remote_kv(shape, seed=11)
    kd, vd = up(k, dtype), up(v, dtype)
    k64, v64 = f64(k, dtype), f64(v, dtype)
    N = S // D
    for r in range(D):
        q = synth.normal((N, H, Dh), 11, synth.TID_Q, r, dtype=dtype)
        o = torch.empty((N, H, Dh), dtype=torch.float32 if odt == "f32" else torch.bfloat16, device="cuda")
        s = tsp.make_shape(S, D, r, H * Dh, H, Dh, 64 * D, dtype=dtype)
        log(f"attention S={S} D={D} r={r} H={H} Dh={Dh} {dtype}->{odt}")
        tsp.tsp_zigzag_attn(s, up(q, dtype), kd, vd, o, tsp.TSP_F32 if odt == "f32" else tsp.TSP_BF16)
        _sync(torch)
        want = oracle.causal_attention(f64(q, dtype), k64, v64, oracle.zigzag_positions(S, D, r), shape.scale)
        got = down(o)
        if dtype == "f32":
            assert_close(got, want, TOL_F32, "o")
        elif odt == "f32":
            assert_close(got, want, TOL_BF16, "o")
        else:
            # a bf16 output adds its own rounding, up to 2^-9 |o| per element
            rms = float(np.sqrt(np.mean(want ** 2)))
            excess = np.abs(got - want) - 2.0 ** -8 * np.abs(want)
            log(f"  o(bf16 out): max excess over rounding = {excess.max():.3e}, rms {rms:.3e}")
            assert excess.max() <= TOL_BF16 * rms


GQA_CASES = [
    # S, D, H, Hkv, Dh, dtype, o_dtype, q pre-scaled
    (2048, 4, 8, 2, 128, "bf16", "f32", False),   # groups of 4 query heads
    (1200, 4, 4, 1, 64, "bf16", "f32", False),    # one K/V head for all (C = 150: ragged tiles)
    (4096, 2, 8, 4, 128, "bf16", "bf16", True),   # the layer's form: Q * scale * log2(e), bf16 O
    (1024, 4, 6, 3, 64, "f32", "f32", False),     # fp32 kernel
]


@pytest.mark.parametrize("S,D,H,Hkv,Dh,dtype,odt,q_log2", GQA_CASES)
def test_grouped_attention(torch, S, D, H, Hkv, Dh, dtype, odt, q_log2):
    """Grouped K/V heads (query head i reads K/V head i // (H/Hkv)) against
    the oracle; every rank."""
    shape = synth.LayerShape(S=S, D=D, h=H * Dh, H=H, Dh=Dh, F=64 * D, dtype=dtype, Hkv=Hkv)
    k, v = synth.remote_kv(shape, seed=17)
    assert k.shape == (S, Hkv, Dh)
    kd, vd = up(k, dtype), up(v, dtype)
    k64, v64 = f64(k, dtype), f64(v, dtype)
    N = S // D
    for r in range(D):
        q = synth.normal((N, H, Dh), 17, synth.TID_Q, r, dtype=dtype)
        s = tsp.make_shape(S, D, r, H * Dh, H, Dh, 64 * D, dtype=dtype, Hkv=Hkv)
        o = torch.empty((N, H, Dh), dtype=torch.float32 if odt == "f32" else torch.bfloat16, device="cuda")
        log(f"grouped attention S={S} D={D} r={r} H={H} Hkv={Hkv} Dh={Dh} {dtype}->{odt} q_log2={q_log2}")
        if q_log2:
            cf = np.float32(s.scale) * np.float32(np.log2(np.e))
            q = synth.f32_to_bf16(synth.bf16_to_f32(q) * cf)
            q64 = f64(q, dtype) / (float(s.scale) * np.log2(np.e))
            tsp.tsp_zigzag_attn_ex(s, up(q, dtype), kd, vd, o, tsp.TSP_BF16, tsp.TSP_ATTN_Q_LOG2_SCALED)
        else:
            q64 = f64(q, dtype)
            tsp.tsp_zigzag_attn(s, up(q, dtype), kd, vd, o, tsp.TSP_F32 if odt == "f32" else tsp.TSP_BF16)
        _sync(torch)
        want = oracle.causal_attention(q64, k64, v64, oracle.zigzag_positions(S, D, r), shape.scale)
        got = down(o)
        if dtype == "f32":
            assert_close(got, want, TOL_F32, "o")
        elif odt == "f32":
            assert_close(got, want, TOL_BF16, "o")
        else:
            rms = float(np.sqrt(np.mean(want ** 2)))
            excess = np.abs(got - want) - 2.0 ** -8 * np.abs(want)
            log(f"  o(bf16 out): max excess over rounding = {excess.max():.3e}, rms {rms:.3e}")
            assert excess.max() <= TOL_BF16 * rms


def test_attention_scale_zero_gives_prefix_mean(torch):
    S, D, H, Dh = 512, 2, 2, 128
    shape = synth.LayerShape(S=S, D=D, h=H * Dh, H=H, Dh=Dh, F=128, dtype="bf16")
    k, v = synth.remote_kv(shape, seed=12)
    q = synth.normal((S // D, H, Dh), 12, synth.TID_Q, 0, dtype="bf16")
    o = torch.empty((S // D, H, Dh), dtype=torch.float32, device="cuda")
    tsp.tsp_zigzag_attn(tsp.make_shape(S, D, 1, H * Dh, H, Dh, 128, scale=0.0), up(q, "bf16"), up(k, "bf16"),
                        up(v, "bf16"), o)
    _sync(torch)
    pos = oracle.zigzag_positions(S, D, 1)
    v64 = f64(v, "bf16")
    want = (np.cumsum(v64, axis=0) / (np.arange(S) + 1)[:, None, None])[pos]
    assert_close(down(o), want, TOL_BF16, "prefix mean")


@pytest.mark.parametrize("Dh,q_log2", [(64, False), (128, False), (64, True), (128, True)])
def test_attention_late_keys_far_above_first_tile(torch, Dh, q_log2):
    """Keys 100, 611 and 1500 get scaled log2 scores of about 16, 24 and 24
    against at most about 5 in any row's first key tile, so the row's
    reference max must move: the kernel raises it on a tile whose
    probabilities (relative to it) sum past 2^16 in some lane. q_log2: Q is
    passed pre-multiplied by scale * log2(e) (TSP_ATTN_Q_LOG2_SCALED, the
    layer's form); the oracle then takes that Q divided by the factor."""
    S, D, H = 2048, 2, 2
    shape = synth.LayerShape(S=S, D=D, h=H * Dh, H=H, Dh=Dh, F=128, dtype="bf16")
    k, v = synth.remote_kv(shape, seed=13)
    kf = synth.bf16_to_f32(k).reshape(S, H, Dh)
    base = np.ones(Dh, dtype=np.float32) / np.sqrt(Dh)
    c = 1.0 / np.sqrt(Dh) * np.log2(np.e)
    for u, lift in ((100, 16.0), (611, 24.0), (1500, 24.0)):
        kf[u] = base * (lift / c) / np.sqrt(Dh) + 0.01 * kf[u]
    k = synth.f32_to_bf16(kf)
    for r in range(D):
        qf = synth.bf16_to_f32(synth.normal((S // D, H, Dh), 13, synth.TID_Q, r, dtype="bf16"))
        qf = qf * 0.05 + base * np.sqrt(Dh)
        q = synth.f32_to_bf16(qf)
        s = tsp.make_shape(S, D, r, H * Dh, H, Dh, 128, dtype="bf16")
        log(f"attention with late large scores Dh={Dh} r={r} q_log2={q_log2}")
        if q_log2:
            cf = np.float32(s.scale) * np.float32(np.log2(np.e))
            q = synth.f32_to_bf16(synth.bf16_to_f32(q) * cf)
            q64 = f64(q, "bf16") / (float(s.scale) * np.log2(np.e))
            o = torch.empty((S // D, H, Dh), dtype=torch.bfloat16, device="cuda")
            tsp.tsp_zigzag_attn_ex(s, up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), o, tsp.TSP_BF16,
                                   tsp.TSP_ATTN_Q_LOG2_SCALED)
        else:
            q64 = f64(q, "bf16")
            o = torch.empty((S // D, H, Dh), dtype=torch.float32, device="cuda")
            tsp.tsp_zigzag_attn(s, up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), o)
        _sync(torch)
        want = oracle.causal_attention(q64, f64(k, "bf16"), f64(v, "bf16"), oracle.zigzag_positions(S, D, r),
                                       shape.scale)
        assert np.isfinite(down(o)).all()
        assert_close(down(o), want, TOL_BF16, "o")


# ---------------------------------------------------------------- MLP ring
MLP_CASES = [
    # S, D, h, F, dtype, residual, MLP form
    (1024, 4, 256, 1024, "f32", False, "gelu"),   # the tiny fp32 layer's MLP
    (1024, 4, 256, 1024, "f32", True, "gelu"),
    (2400, 4, 512, 2048, "bf16", True, "gelu"),   # N = 600: ragged row tiles
    (2048, 2, 256, 512, "bf16", False, "gelu"),
    (1024, 1, 256, 256, "bf16", False, "gelu"),   # D = 1
    (4096, 8, 640, 1024, "bf16", True, "gelu"),   # N = 512, h not a multiple of the tile
    (1024, 4, 256, 1024, "f32", True, "swiglu"),  # gated: (gate, up) column pairs
    (2400, 4, 512, 2048, "bf16", True, "swiglu"),  # gated: 64 gate + 64 up columns per 128, ragged rows
    (1024, 2, 256, 128, "bf16", False, "swiglu"),  # gated, F/D = 64: 128 product columns, half a tile
    (4096, 8, 640, 1024, "bf16", True, "swiglu"),
    (1024, 1, 192, 192, "bf16", True, "gelu"),    # 3 K steps in both products (odd: the loop's lone last step)
    (1152, 3, 64, 192, "bf16", True, "gelu"),     # 1 K step in the up product; down: 3 steps, a new shard each
    (1024, 1, 192, 192, "bf16", False, "swiglu"),  # gated, 3 K steps
]


@pytest.mark.parametrize("S,D,h,F,dtype,resid,mlp", MLP_CASES)
def test_mlp_ring(torch, S, D, h, F, dtype, resid, mlp):
    shape = synth.LayerShape(S=S, D=D, h=h, H=h // 64, Dh=64, F=F, dtype=dtype, mlp=mlp)
    N = S // D
    w = synth.layer_weights(shape, seed=21)
    x = synth.activations(N, h, seed=21, dtype=dtype)
    res = synth.activations(N, h, seed=22) if resid else None
    w1d = [up(a, dtype) for a in w["w1"]]
    w2d = [up(a, dtype) for a in w["w2"]]
    xd = up(x, dtype)
    want = oracle.mlp(f64(x, dtype), [f64(a, dtype) for a in w["w1"]], [f64(a, dtype) for a in w["w2"]],
                      gated=mlp == "swiglu")
    if resid:
        want = want + res.astype(np.float64)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    outs = []
    for r in sorted({0, D - 1, D // 2}):
        s = tsp.make_shape(S, D, r, h, h // 64, 64, F, dtype=dtype, mlp=mlp)
        ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_MLP), dtype=torch.uint8, device="cuda")
        y = torch.full((N, h), float("nan"), dtype=torch.float32, device="cuda")
        log(f"mlp ring S={S} D={D} r={r} h={h} F={F} {dtype} residual={resid} {mlp}")
        tsp.tsp_mlp_ring(s, xd, w1d, w2d, up(res, "f32") if resid else None, y, ws)
        _sync(torch)
        outs.append(down(y))
        assert_close(outs[-1], want, tol, "y")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gelu_through_identity_mlp(torch, dtype):
    """With D = 1 and W1 = W2 = I the ring returns GELU(x) itself (identity
    products are exact), so the kernels' GELU is checked value by value
    against the erf definition over z in [-10, 10]."""
    S, D, h = 8192, 1, 64
    N = S // D
    z = np.linspace(-10.0, 10.0, N * h).astype(np.float32).reshape(N, h)
    eye = np.eye(h, dtype=np.float32)
    if dtype == "bf16":
        zq = synth.f32_to_bf16(z)
        zin, z64 = up(zq, "bf16"), synth.bf16_to_f32(zq).astype(np.float64)
        w1, w2 = up(synth.f32_to_bf16(eye), "bf16"), up(synth.f32_to_bf16(eye), "bf16")
    else:
        zin, z64 = up(z, "f32"), z.astype(np.float64)
        w1, w2 = up(eye, "f32"), up(eye, "f32")
    s = tsp.make_shape(S, D, 0, h, 1, 64, h, dtype=dtype)
    ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_MLP), dtype=torch.uint8, device="cuda")
    y = torch.empty((N, h), dtype=torch.float32, device="cuda")
    tsp.tsp_mlp_ring(s, zin, [w1], [w2], None, y, ws)
    _sync(torch)
    want = oracle.gelu(z64)
    err = np.abs(down(y) - want)
    if dtype == "f32":
        bound = 1e-6 * np.maximum(1.0, np.abs(z64))
    else:
        bound = 2.0 ** -8 * np.abs(want) + 1e-6 * np.maximum(1.0, np.abs(z64))  # H is rounded to bf16
    log(f"GELU {dtype}: max |err| = {err.max():.3e}, max err/bound = {(err / bound).max():.3f}")
    assert (err <= bound).all()


def test_mlp_ring_residual_in_place(torch):
    S, D, h, F = 1024, 4, 256, 1024
    shape = synth.LayerShape(S=S, D=D, h=h, H=4, Dh=64, F=F, dtype="bf16")
    w = synth.layer_weights(shape, seed=23)
    x = synth.activations(S // D, h, seed=23, dtype="bf16")
    res = synth.activations(S // D, h, seed=24)
    s = tsp.make_shape(S, D, 2, h, 4, 64, F, dtype="bf16")
    ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_MLP), dtype=torch.uint8, device="cuda")
    y = up(res, "f32")
    tsp.tsp_mlp_ring(s, up(x, "bf16"), [up(a, "bf16") for a in w["w1"]], [up(a, "bf16") for a in w["w2"]], y, y, ws)
    _sync(torch)
    want = res + oracle.mlp(f64(x, "bf16"), [f64(a, "bf16") for a in w["w1"]], [f64(a, "bf16") for a in w["w2"]])
    assert_close(down(y), want, TOL_BF16, "y (residual == y)")


# ---------------------------------------------------------------- whole layer
def _dev_weights(w, dtype):
    return {k: ([up(a, dtype) for a in w[k]] if isinstance(w[k], list) else up(w[k], dtype))
            for k in ("wqkv", "wo", "w1", "w2", "g_attn", "g_mlp")}


def _w64(w, dtype):
    return {k: ([f64(a, dtype) for a in w[k]] if isinstance(w[k], list) else f64(w[k], dtype)) for k in w}


@pytest.mark.parametrize("gain,rope", [("ones", 0.0), ("random", 0.0), ("random", 10000.0)])
def test_tiny_layer_every_rank_vs_unsharded(torch, gain, rope):
    """Tiny fp32 layer (S=1024, D=4, h=256, 4 heads of 64, F=1024): the D ranks
    each write their K/V rows into one shared buffer (the all-gather), then each
    runs the rest; every rank's rows must equal the unsharded layer's. rope:
    rotary base (0 = none)."""
    shape = synth.TINY_FP32
    S, D, h, H, Dh, F = shape.S, shape.D, shape.h, shape.H, shape.Dh, shape.F
    w = synth.layer_weights(shape, seed=1, gain=gain)
    x_full = synth.activations(S, h, seed=1)
    full = oracle.layer_full(x_full, _w64(w, "f32"), H, Dh, shape.eps, shape.scale, rope_base=rope)
    wd = _dev_weights(w, "f32")
    kf = torch.zeros((S, H, Dh), dtype=torch.float32, device="cuda")
    vf = torch.zeros_like(kf)
    ranks = []
    for r in range(D):
        s = tsp.make_shape(S, D, r, h, H, Dh, F, eps=shape.eps, dtype="f32", rope_base=rope)
        pos = oracle.zigzag_positions(S, D, r)
        ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")
        xd = up(x_full[pos], "f32")
        y = torch.full((S // D, h), float("nan"), dtype=torch.float32, device="cuda")
        tsp.tsp_layer_fwd(s, wd, xd, kf, vf, y, tsp.TSP_PHASE_KV, ws)
        ranks.append((s, pos, ws, xd, y))
    for s, pos, ws, xd, y in ranks:
        tsp.tsp_layer_fwd(s, wd, xd, kf, vf, y, tsp.TSP_PHASE_REST, ws)
    _sync(torch)
    assert_close(down(kf), full["k"], TOL_F32, "gathered K")
    assert_close(down(vf), full["v"], TOL_F32, "gathered V")
    got = np.zeros_like(full["y"])
    for s, pos, ws, xd, y in ranks:
        got[pos] = down(y)
        log(f"rank {s.r}:")
        assert_close(down(y), full["y"][pos], TOL_F32, "y rows")
    assert_close(got, full["y"], TOL_F32, "y, all ranks")


@pytest.mark.parametrize("rope,mlp", [(0.0, "gelu"), (10000.0, "gelu"), (10000.0, "swiglu")])
def test_fp32_grouped_layer_every_rank_vs_unsharded(torch, rope, mlp):
    """fp32 layer with 8 query heads sharing 2 K/V heads (S=1024, D=2, h=512,
    Dh=64, F=1024): the ranks write their K/V rows into one gathered buffer of
    2 heads, then each runs the rest; every rank's rows must equal the
    unsharded grouped layer's. Also with rotation, and with the gated MLP."""
    S, D, H, Hkv, Dh, F = 1024, 2, 8, 2, 64, 1024
    h = H * Dh
    shape = synth.LayerShape(S=S, D=D, h=h, H=H, Dh=Dh, F=F, dtype="f32", Hkv=Hkv, mlp=mlp)
    w = synth.layer_weights(shape, seed=5, gain="random")
    assert w["wqkv"][0].shape == ((H + 2 * Hkv) * Dh // D, h)
    x_full = synth.activations(S, h, seed=5)
    full = oracle.layer_full(x_full, _w64(w, "f32"), H, Dh, shape.eps, shape.scale, rope_base=rope, Hkv=Hkv,
                             gated=mlp == "swiglu")
    wd = _dev_weights(w, "f32")
    kf = torch.zeros((S, Hkv, Dh), dtype=torch.float32, device="cuda")
    vf = torch.zeros_like(kf)
    ranks = []
    for r in range(D):
        s = tsp.make_shape(S, D, r, h, H, Dh, F, eps=shape.eps, dtype="f32", rope_base=rope, Hkv=Hkv, mlp=mlp)
        pos = oracle.zigzag_positions(S, D, r)
        ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")
        xd = up(x_full[pos], "f32")
        y = torch.full((S // D, h), float("nan"), dtype=torch.float32, device="cuda")
        log(f"fp32 grouped layer r={r} rope={rope} {mlp}: K/V phase")
        tsp.tsp_layer_fwd(s, wd, xd, kf, vf, y, tsp.TSP_PHASE_KV, ws)
        ranks.append((s, pos, ws, xd, y))
    for s, pos, ws, xd, y in ranks:
        tsp.tsp_layer_fwd(s, wd, xd, kf, vf, y, tsp.TSP_PHASE_REST, ws)
    _sync(torch)
    assert_close(down(kf), full["k"], TOL_F32, "gathered K")
    assert_close(down(vf), full["v"], TOL_F32, "gathered V")
    for s, pos, ws, xd, y in ranks:
        log(f"rank {s.r}:")
        assert_close(down(y), full["y"][pos], TOL_F32, "y rows")


def test_tiny_layer_rank_mode_given_remote_kv(torch):
    shape = synth.TINY_FP32
    S, D, h, H, Dh, F = shape.S, shape.D, shape.h, shape.H, shape.Dh, shape.F
    w = synth.layer_weights(shape, seed=2, gain="random")
    w64 = _w64(w, "f32")
    wd = _dev_weights(w, "f32")
    k_rem, v_rem = synth.remote_kv(shape, seed=2)
    for r in range(D):
        x = synth.activations(S // D, h, seed=2, tid=100 + r)
        s = tsp.make_shape(S, D, r, h, H, Dh, F, eps=shape.eps, dtype="f32")
        ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")
        kf, vf = up(k_rem, "f32"), up(v_rem, "f32")
        y = torch.empty((S // D, h), dtype=torch.float32, device="cuda")
        tsp.tsp_layer_fwd(s, wd, up(x, "f32"), kf, vf, y, tsp.TSP_PHASE_ALL, ws)
        _sync(torch)
        want = oracle.layer_rank(x, w64, k_rem, v_rem, S, D, r, H, Dh, shape.eps, shape.scale)
        log(f"rank {r}:")
        assert_close(down(y), want["y"], TOL_F32, "y")
        assert_close(down(y) - x, want["y"] - x, 10 * TOL_F32, "y - x (both branches)")


@pytest.mark.parametrize("S,D,H,Dh,F,rope,Hkv,mlp", [
    (2048, 4, 4, 128, 2048, 0.0, 0, "gelu"),
    (2400, 4, 4, 128, 2048, 0.0, 0, "gelu"),   # N = 600: ragged row tiles
    (1024, 2, 4, 64, 1024, 0.0, 0, "gelu"),
    (96, 3, 6, 64, 576, 0.0, 0, "gelu"),       # C = 16: rank 0 recomputes 16 leading rows (one 32-row MFMA block)
    (256, 1, 4, 64, 512, 0.0, 0, "gelu"),      # D = 1: one shard, the plain layer
    (2048, 4, 4, 128, 2048, 10000.0, 0, "gelu"),  # rotary embedding, heads of 128
    (1024, 2, 4, 64, 1024, 500.0, 0, "gelu"),     # rotary embedding, heads of 64 (two per 128-column block)
    (96, 3, 6, 64, 576, 10000.0, 0, "gelu"),      # rotary embedding on the 16 leading rows too
    (2048, 4, 8, 128, 2048, 0.0, 4, "gelu"),      # grouped K/V: 2 query heads per K/V head, 128-column blocks
    (2048, 4, 8, 128, 2048, 10000.0, 4, "gelu"),  # grouped K/V with rotation in the epilogue
    (1024, 2, 4, 64, 1024, 0.0, 2, "gelu"),       # grouped K/V, 64-column K/V parts (element-wise epilogue)
    (96, 3, 6, 64, 576, 0.0, 3, "gelu"),          # grouped K/V on the 16 leading rows
    (96, 3, 6, 128, 576, 10000.0, 3, "gelu"),     # grouped K/V and rotation on the 16 leading rows, heads of 128
    (2048, 4, 4, 128, 2048, 0.0, 0, "swiglu"),      # gated MLP
    (96, 3, 6, 64, 576, 0.0, 0, "swiglu"),          # gated MLP on the 16 leading rows
    (2048, 4, 8, 128, 2048, 10000.0, 4, "swiglu"),  # rotation, grouped K/V and the gated MLP together
    (192, 3, 3, 64, 192, 0.0, 0, "gelu"),    # h = 192: 3 K steps in every product, a new W_O / W2 shard every step
    (192, 3, 3, 64, 192, 0.0, 0, "swiglu"),  # the same with the gated MLP
])
def test_bf16_layer_vs_oracle(torch, S, D, H, Dh, F, rope, Hkv, mlp):
    h = H * Dh
    shape = synth.LayerShape(S=S, D=D, h=h, H=H, Dh=Dh, F=F, dtype="bf16", Hkv=Hkv, mlp=mlp)
    gated = mlp == "swiglu"
    w = synth.layer_weights(shape, seed=3, gain="random")
    w64 = _w64(w, "bf16")
    wd = _dev_weights(w, "bf16")
    k_rem, v_rem = synth.remote_kv(shape, seed=3)
    k64, v64 = f64(k_rem, "bf16"), f64(v_rem, "bf16")
    for r in sorted({0, D - 1}):
        x = synth.activations(S // D, h, seed=3, tid=100 + r)
        s = tsp.make_shape(S, D, r, h, H, Dh, F, eps=shape.eps, dtype="bf16", rope_base=rope, Hkv=Hkv, mlp=mlp)
        ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")
        kf, vf = up(k_rem, "bf16"), up(v_rem, "bf16")
        y = torch.empty((S // D, h), dtype=torch.float32, device="cuda")
        log(f"bf16 layer S={S} D={D} r={r} H={H} Hkv={Hkv} Dh={Dh} F={F} rope={rope} {mlp}")
        tsp.tsp_layer_fwd(s, wd, up(x, "f32"), kf, vf, y, tsp.TSP_PHASE_ALL, ws)
        _sync(torch)
        want = oracle.layer_rank(x, w64, k64, v64, S, D, r, H, Dh, shape.eps, shape.scale, rope_base=rope,
                                 Hkv=Hkv or None, gated=gated)
        err = assert_close(down(y), want["y"], TOL_BF16, "y")
        if rope > 0:
            # the output is much closer to the rotated layer than to the plain one
            plain = oracle.layer_rank(x, w64, k64, v64, S, D, r, H, Dh, shape.eps, shape.scale, Hkv=Hkv or None,
                                      gated=gated)["y"]
            far = float(np.abs(down(y) - plain).max()) / float(np.sqrt(np.mean(want["y"] ** 2)))
            log(f"  distance to the layer without rotation: {far:.3e} rms")
            assert far > 5 * err
        if r == 0:
            # rank 0's first positions are recomputed with fp32 intermediates
            m = min(64, S // (2 * D))
            assert_close(down(y)[:m], want["y"][:m], TOL_F32, f"leading {m} rows")
        # remote rows of the gathered K/V are left untouched
        pos = oracle.zigzag_positions(S, D, r)
        remote = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(kf.view(torch.int16).cpu().numpy()[remote], k_rem.view(np.int16)[remote])


def test_layer_deterministic(torch):
    S, D, H, Dh, F = 2048, 4, 4, 128, 2048
    h = H * Dh
    shape = synth.LayerShape(S=S, D=D, h=h, H=H, Dh=Dh, F=F, dtype="bf16")
    w = synth.layer_weights(shape, seed=4)
    wd = _dev_weights(w, "bf16")
    k_rem, v_rem = synth.remote_kv(shape, seed=4)
    x = up(synth.activations(S // D, h, seed=4), "f32")
    s = tsp.make_shape(S, D, 1, h, H, Dh, F, dtype="bf16")
    outs = []
    for _ in range(2):
        ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")
        y = torch.empty((S // D, h), dtype=torch.float32, device="cuda")
        tsp.tsp_layer_fwd(s, wd, x, up(k_rem, "bf16"), up(v_rem, "bf16"), y, tsp.TSP_PHASE_ALL, ws)
        _sync(torch)
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("dtype,layers,S,D,H,Dh,F", [("f32", 32, 1024, 4, 4, 64, 1024),
                                                      ("bf16", 4, 2400, 4, 4, 128, 2048)])
def test_layer_stack_vs_oracle(torch, dtype, layers, S, D, H, Dh, F):
    """A stack of layers on one rank's share (the 32-layer 7B forward at small
    size): layer l reads layer l-1's output and has its own seeded weights
    and remote K/V. The oracle runs the same stack in fp64 on its own
    intermediate results."""
    h = H * Dh
    shape = synth.LayerShape(S=S, D=D, h=h, H=H, Dh=Dh, F=F, dtype=dtype)
    r = D - 1
    s = tsp.make_shape(S, D, r, h, H, Dh, F, eps=shape.eps, dtype=dtype)
    ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")
    x0 = synth.activations(S // D, h, seed=5, tid=100 + r)
    bufs = [up(x0, "f32"), torch.empty((S // D, h), dtype=torch.float32, device="cuda")]
    want = x0.astype(np.float64)
    keep = []
    for l in range(layers):
        w = synth.layer_weights(shape, seed=500 + l, gain="random")
        k_rem, v_rem = synth.remote_kv(shape, seed=500 + l)
        kf, vf = up(k_rem, dtype), up(v_rem, dtype)
        wd = _dev_weights(w, dtype)
        keep.append((wd, kf, vf))
        tsp.tsp_layer_fwd(s, wd, bufs[l % 2], kf, vf, bufs[(l + 1) % 2], tsp.TSP_PHASE_ALL, ws)
        want = oracle.layer_rank(want, _w64(w, dtype), f64(k_rem, dtype), f64(v_rem, dtype), S, D, r, H, Dh,
                                 shape.eps, shape.scale)["y"]
    _sync(torch)
    log(f"{layers}-layer stack S={S} D={D} r={r} {dtype}")
    assert_close(down(bufs[layers % 2]), want, TOL_F32 if dtype == "f32" else TOL_BF16, "y after the stack")
