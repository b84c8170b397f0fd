"""GPU parity of the MLP ring backward (tsp_mlp_ring_bwd) against the fp64
oracle's chain-rule gradients: small shapes in both dtypes on every rank
(ragged tiles, shards narrower than a tile, the residual in place), the D
ranks' weight-gradient contributions summed against the gradient over the
whole sequence, and the 7B shape with sampled rows of dx and sampled hidden
units of dW1 and dW2."""
import numpy as np
import pytest

import oracle
import synth
import tsp_rank_local_amd as tsp
from gpu_util import TOL_BF16, TOL_F32, assert_close, assert_close_nw, down, f64, log, torch_cuda, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_cuda()
    tsp.lib()
    return t


def _run(torch, s, x, w1, w2, dy, res=None, in_place=False):
    """Calls tsp_mlp_ring_bwd; returns dx, dw1, dw2 as float64 numpy (dw lists by shard)."""
    D, N, h, fd = s.D, s.S // s.D, s.h, s.F // s.D
    ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_MLP_BWD), dtype=torch.uint8, device="cuda")
    if in_place:
        dx = res.clone()
        resd = dx
    else:
        dx = torch.full((N, h), float("nan"), dtype=torch.float32, device="cuda")
        resd = res
    dw1 = [torch.full((fd, h), float("nan"), dtype=torch.float32, device="cuda") for _ in range(D)]
    dw2 = [torch.full((h, fd), float("nan"), dtype=torch.float32, device="cuda") for _ in range(D)]
    tsp.tsp_mlp_ring_bwd(s, x, w1, w2, dy, resd, dx, dw1, dw2, ws)
    torch.cuda.synchronize()
    return down(dx), [down(a) for a in dw1], [down(a) for a in dw2]


def _check(got, want, tol, tag):
    dx, dw1, dw2 = got
    assert_close(dx, want["dx"], tol, f"dx {tag}")
    assert_close(np.concatenate(dw1, axis=0), np.concatenate(want["dw1"], axis=0), tol, f"dW1 {tag}")
    assert_close(np.concatenate(dw2, axis=1), np.concatenate(want["dw2"], axis=1), tol, f"dW2 {tag}")


BWD_CASES = [
    # S, D, h, F, dtype
    (1024, 4, 256, 1024, "f32"),   # the tiny fp32 layer's MLP
    (2048, 4, 256, 1024, "bf16"),  # 512 tokens: two token tiles
    (640, 2, 320, 384, "bf16"),    # 320 tokens, h = 320, F/D = 192: ragged tiles, shard not a multiple of 128
    (1024, 8, 192, 512, "bf16"),   # F/D = 64: half a tile of hidden units per shard
    (128, 1, 64, 64, "bf16"),      # D = 1, one tile everywhere
]


@pytest.mark.parametrize("S,D,h,F,dtype", BWD_CASES)
def test_mlp_ring_bwd_every_rank(torch, S, D, h, F, dtype):
    shape = synth.LayerShape(S=S, D=D, h=h, H=h // 64, Dh=64, F=F, dtype=dtype)
    N = S // D
    w = synth.layer_weights(shape, seed=41)
    x = synth.activations(N, h, seed=41, dtype=dtype)
    dy = synth.activations(N, h, seed=41, tid=synth.TID_DY, dtype=dtype)
    w1d, w2d = [up(a, dtype) for a in w["w1"]], [up(a, dtype) for a in w["w2"]]
    want = oracle.mlp_backward(f64(x, dtype), [f64(a, dtype) for a in w["w1"]], [f64(a, dtype) for a in w["w2"]],
                               f64(dy, dtype))
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    for r in range(D):
        s = tsp.make_shape(S, D, r, h, h // 64, 64, F, dtype=dtype)
        log(f"mlp ring bwd S={S} D={D} r={r} h={h} F={F} {dtype}")
        _check(_run(torch, s, up(x, dtype), w1d, w2d, up(dy, dtype)), want, tol, f"r={r}")


@pytest.mark.parametrize("S,D,h,F", [(2048, 4, 256, 1024), (640, 2, 320, 384), (128, 1, 64, 64)])
def test_mlp_ring_z_and_bwd_from_forward(torch, S, D, h, F):
    """tsp_mlp_ring_z (y and the pre-activation Z in ring-step columns) and
    tsp_mlp_ring_bwd_z taking that Z, every rank, bf16, against the oracle."""
    shape = synth.LayerShape(S=S, D=D, h=h, H=h // 64, Dh=64, F=F, dtype="bf16")
    N, fd = S // D, F // D
    w = synth.layer_weights(shape, seed=46)
    x = synth.activations(N, h, seed=46, dtype="bf16")
    dy = synth.activations(N, h, seed=46, tid=synth.TID_DY, dtype="bf16")
    w1_64, w2_64 = [f64(a, "bf16") for a in w["w1"]], [f64(a, "bf16") for a in w["w2"]]
    x64 = f64(x, "bf16")
    want_y = oracle.mlp(x64, w1_64, w2_64)
    want = oracle.mlp_backward(x64, w1_64, w2_64, f64(dy, "bf16"))
    xd, dyd = up(x, "bf16"), up(dy, "bf16")
    w1d, w2d = [up(a, "bf16") for a in w["w1"]], [up(a, "bf16") for a in w["w2"]]
    for r in range(D):
        s = tsp.make_shape(S, D, r, h, h // 64, 64, F, dtype="bf16")
        log(f"mlp ring with Z, then backward from it: S={S} D={D} r={r} h={h} F={F}")
        ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_MLP), dtype=torch.uint8, device="cuda")
        y = torch.empty((N, h), dtype=torch.float32, device="cuda")
        z = torch.empty((N, F), dtype=torch.bfloat16, device="cuda")
        tsp.tsp_mlp_ring_z(s, xd, w1d, w2d, None, y, z, ws)
        torch.cuda.synchronize()
        assert_close(down(y), want_y, TOL_BF16, f"y r={r}")
        # ring step t holds shard (r - t) mod D in columns t*fd..
        want_z = np.concatenate([x64 @ w1_64[(r - t) % D].T for t in range(D)], axis=1)
        assert_close(down(z), want_z, TOL_BF16, f"Z r={r}")
        wsb = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_MLP_BWD), dtype=torch.uint8, device="cuda")
        dx = torch.full((N, h), float("nan"), dtype=torch.float32, device="cuda")
        dw1 = [torch.full((fd, h), float("nan"), dtype=torch.float32, device="cuda") for _ in range(D)]
        dw2 = [torch.full((h, fd), float("nan"), dtype=torch.float32, device="cuda") for _ in range(D)]
        tsp.tsp_mlp_ring_bwd_z(s, xd, z, w1d, w2d, dyd, None, dx, dw1, dw2, wsb)
        torch.cuda.synchronize()
        _check((down(dx), [down(a) for a in dw1], [down(a) for a in dw2]), want, TOL_BF16, f"from Z, r={r}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mlp_ring_bwd_residual_in_place(torch, dtype):
    S, D, h, F = 1024, 4, 256, 1024
    shape = synth.LayerShape(S=S, D=D, h=h, H=4, Dh=64, F=F, dtype=dtype)
    N = S // D
    w = synth.layer_weights(shape, seed=42)
    x = synth.activations(N, h, seed=42, dtype=dtype)
    dy = synth.activations(N, h, seed=42, tid=synth.TID_DY, dtype=dtype)
    res = synth.activations(N, h, seed=43)
    want = oracle.mlp_backward(f64(x, dtype), [f64(a, dtype) for a in w["w1"]], [f64(a, dtype) for a in w["w2"]],
                               f64(dy, dtype))
    want["dx"] = want["dx"] + res.astype(np.float64)
    s = tsp.make_shape(S, D, 1, h, 4, 64, F, dtype=dtype)
    log(f"mlp ring bwd residual == dx, {dtype}")
    got = _run(torch, s, up(x, dtype), [up(a, dtype) for a in w["w1"]], [up(a, dtype) for a in w["w2"]],
               up(dy, dtype), up(res, "f32"), in_place=True)
    _check(got, want, TOL_F32 if dtype == "f32" else TOL_BF16, "residual")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mlp_ring_bwd_rank_contributions_sum(torch, dtype):
    """D emulated ranks, each on its own zigzag tokens of one sequence: every
    rank's dx rows are the full-sequence dx at its positions, and the ranks'
    weight-gradient contributions add up to the whole sequence's gradient."""
    S, D, h, F = 2048, 4, 256, 512
    shape = synth.LayerShape(S=S, D=D, h=h, H=4, Dh=64, F=F, dtype=dtype)
    w = synth.layer_weights(shape, seed=44)
    x = synth.activations(S, h, seed=44, dtype=dtype)
    dy = synth.activations(S, h, seed=44, tid=synth.TID_DY, dtype=dtype)
    w1_64, w2_64 = [f64(a, dtype) for a in w["w1"]], [f64(a, dtype) for a in w["w2"]]
    full = oracle.mlp_backward(f64(x, dtype), w1_64, w2_64, f64(dy, dtype))
    w1d, w2d = [up(a, dtype) for a in w["w1"]], [up(a, dtype) for a in w["w2"]]
    acc1 = [np.zeros_like(a) for a in full["dw1"]]
    acc2 = [np.zeros_like(a) for a in full["dw2"]]
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        s = tsp.make_shape(S, D, r, h, 4, 64, F, dtype=dtype)
        log(f"mlp ring bwd, emulated rank {r} of {D}, {dtype}")
        dx, dw1, dw2 = _run(torch, s, up(x[pos], dtype), w1d, w2d, up(dy[pos], dtype))
        assert_close(dx, full["dx"][pos], tol, f"dx rows of rank {r}")
        for j in range(D):
            acc1[j] += dw1[j]
            acc2[j] += dw2[j]
    assert_close(np.concatenate(acc1, axis=0), np.concatenate(full["dw1"], axis=0), tol, "sum of dW1 contributions")
    assert_close(np.concatenate(acc2, axis=1), np.concatenate(full["dw2"], axis=1), tol, "sum of dW2 contributions")


@pytest.mark.timeout(900)
def test_mlp_ring_bwd_7b(torch):
    """7B shape (16384 tokens, h 4096, F 16384, D 8), ring starts r = 0 and 5:
    dx on 64 strided rows (each needs its whole hidden row), dW1 rows and dW2
    columns of 48 strided hidden units (each needs that unit's pre-activation
    over all tokens), against the oracle's chain rule on those slices."""
    SH = synth.SEVEN_B
    N, h, F, D = SH.N, SH.h, SH.F, SH.D
    fd = F // D
    w = synth.layer_weights(SH, seed=45)
    x = synth.activations(N, h, seed=45, dtype="bf16")
    dy = synth.activations(N, h, seed=45, tid=synth.TID_DY, dtype="bf16")
    x64, dy64 = f64(x, "bf16"), f64(dy, "bf16")
    W1 = np.concatenate([f64(a, "bf16") for a in w["w1"]], axis=0)
    W2 = np.concatenate([f64(a, "bf16") for a in w["w2"]], axis=1)
    rows = np.linspace(0, N - 1, 64).round().astype(np.int64)
    units = np.linspace(0, F - 1, 48).round().astype(np.int64)
    # dx rows: the oracle on those tokens alone (each token's dx depends only on its own x and dy)
    want_dx = oracle.mlp_backward(x64[rows], [f64(a, "bf16") for a in w["w1"]],
                                  [f64(a, "bf16") for a in w["w2"]], dy64[rows])["dx"]
    # hidden units: Z[:, f], GELU and GELU' over all tokens, written from the chain rule
    Zu = x64 @ W1[units].T
    dZu = (dy64 @ W2[:, units]) * oracle.gelu_grad(Zu)
    want_dw1 = dZu.T @ x64             # [units, h]
    want_dw2 = dy64.T @ oracle.gelu(Zu)  # [h, units]
    xd, dyd = up(x, "bf16"), up(dy, "bf16")
    w1d, w2d = [up(a, "bf16") for a in w["w1"]], [up(a, "bf16") for a in w["w2"]]
    for r in (0, 5):
        s = tsp.make_shape(SH.S, D, r, h, SH.H, SH.Dh, F, dtype="bf16")
        log(f"mlp ring bwd 7B, ring start r={r}")
        dx, dw1, dw2 = _run(torch, s, xd, w1d, w2d, dyd)
        assert_close(dx[rows], want_dx, TOL_BF16, f"dx rows (r={r})")
        g1 = np.stack([dw1[u // fd][u % fd] for u in units])
        g2 = np.stack([dw2[u // fd][:, u % fd] for u in units], axis=1)
        assert_close(g1, want_dw1, TOL_BF16, f"dW1 rows of sampled units (r={r})")
        assert_close(g2, want_dw2, TOL_BF16, f"dW2 columns of sampled units (r={r})")
        assert all(np.isfinite(a).all() for a in dw1 + dw2) and np.isfinite(dx).all()


# ---------------------------------------------------------------- attention backward
def _attn_bwd_run(torch, s, q, k, v, do, dtype, from_fwd=False, flags=None):
    """tsp_zigzag_attn_bwd, or (from_fwd) tsp_zigzag_attn_lse followed by
    tsp_zigzag_attn_bwd_lse; with flags, tsp_zigzag_attn_bwd_ex (statistics
    from the forward when from_fwd); returns dq, dk, dv (float64)."""
    N, H, Dh = q.shape
    S, Hkv = k.shape[0], k.shape[1]
    qd, kd, vd, dod = up(q, dtype), up(k, dtype), up(v, dtype), up(do, dtype)
    if from_fwd:
        o = torch.empty((N, H, Dh), dtype=torch.float32, device="cuda")
        lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
        tsp.tsp_zigzag_attn_lse(s, qd, kd, vd, o, lse)
    ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_ATTN_BWD), dtype=torch.uint8, device="cuda")
    dq = torch.full((N, H, Dh), float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.full((S, Hkv, Dh), float("nan"), dtype=torch.float32, device="cuda")
    dv = torch.full((S, Hkv, Dh), float("nan"), dtype=torch.float32, device="cuda")
    if flags is not None:
        tsp.tsp_zigzag_attn_bwd_ex(s, qd, kd, vd, o if from_fwd else None, lse if from_fwd else None, dod, dq, dk,
                                   dv, flags, ws)
    elif from_fwd:
        tsp.tsp_zigzag_attn_bwd_lse(s, qd, kd, vd, o, lse, dod, dq, dk, dv, ws)
    else:
        tsp.tsp_zigzag_attn_bwd(s, qd, kd, vd, dod, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return down(dq), down(dk), down(dv)


ATTN_BWD_CASES = [
    # S, D, H, Hkv, Dh, dtype
    (1024, 4, 4, 4, 64, "f32"),    # the tiny fp32 layer's attention
    (2048, 4, 4, 4, 128, "bf16"),  # chunks of 256: two query tiles, eight 32-row steps each
    (640, 2, 2, 2, 64, "bf16"),    # chunks of 160: a ragged query tile and step
    (1024, 2, 4, 2, 128, "bf16"),  # two query heads per K/V head
    (256, 1, 2, 2, 128, "bf16"),   # D = 1: plain causal attention
    # chunks of 100: the dK/dV walks (16 to 100 rows) end inside a 32-row
    # step and inside a 64-row stage
    (600, 3, 3, 3, 64, "bf16"),
    (600, 3, 6, 3, 128, "bf16"),   # and two query heads per K/V head: a walk per head
]


@pytest.mark.parametrize("S,D,H,Hkv,Dh,dtype", ATTN_BWD_CASES)
def test_attn_bwd_every_rank(torch, S, D, H, Hkv, Dh, dtype):
    shape = synth.LayerShape(S=S, D=D, h=H * Dh, H=H, Dh=Dh, F=64 * D, dtype=dtype, Hkv=Hkv)
    N = S // D
    k, v = synth.remote_kv(shape, seed=51)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    for r in range(D):
        q = synth.normal((N, H, Dh), 51, synth.TID_Q, r, dtype=dtype)
        do = synth.normal((N, H, Dh), 51, synth.TID_DY, r, dtype=dtype)
        pos = oracle.zigzag_positions(S, D, r)
        want = oracle.causal_attention_backward(f64(q, dtype), f64(k, dtype), f64(v, dtype), pos, shape.scale,
                                                f64(do, dtype))
        s = tsp.make_shape(S, D, r, H * Dh, H, Dh, 64 * D, dtype=dtype, Hkv=Hkv)
        log(f"attention backward S={S} D={D} r={r} H={H} Hkv={Hkv} Dh={Dh} {dtype}")
        dq, dk, dv = _attn_bwd_run(torch, s, q, k, v, do, dtype)
        assert_close(dq, want["dq"], tol, f"dq r={r}")
        assert_close(dk, want["dk"], tol, f"dk r={r}")
        assert_close(dv, want["dv"], tol, f"dv r={r}")
        assert not dk[pos.max() + 1:].any() and not dv[pos.max() + 1:].any()


@pytest.mark.parametrize("S,D,H,Hkv,Dh,dtype", [c for c in ATTN_BWD_CASES if c[-1] == "bf16"])
def test_attn_lse_and_bwd_from_forward_every_rank(torch, S, D, H, Hkv, Dh, dtype):
    """tsp_zigzag_attn_lse (fp32 O and the row log-sum-exp) and the backward
    that takes them, on every rank, against the oracle."""
    shape = synth.LayerShape(S=S, D=D, h=H * Dh, H=H, Dh=Dh, F=64 * D, dtype=dtype, Hkv=Hkv)
    N = S // D
    k, v = synth.remote_kv(shape, seed=51)
    k64, v64 = f64(k, dtype), f64(v, dtype)
    for r in range(D):
        q = synth.normal((N, H, Dh), 51, synth.TID_Q, r, dtype=dtype)
        do = synth.normal((N, H, Dh), 51, synth.TID_DY, r, dtype=dtype)
        pos = oracle.zigzag_positions(S, D, r)
        s = tsp.make_shape(S, D, r, H * Dh, H, Dh, 64 * D, dtype=dtype, Hkv=Hkv)
        log(f"attention with log-sum-exp, then backward from it: S={S} D={D} r={r} H={H} Hkv={Hkv} Dh={Dh}")
        o = torch.empty((N, H, Dh), dtype=torch.float32, device="cuda")
        lse = torch.full((H, N), float("nan"), dtype=torch.float32, device="cuda")
        tsp.tsp_zigzag_attn_lse(s, up(q, dtype), up(k, dtype), up(v, dtype), o, lse)
        torch.cuda.synchronize()
        want_lse = oracle.causal_attention_lse(f64(q, dtype), k64, pos, shape.scale)
        err = float(np.abs(down(lse) - want_lse).max())
        log(f"  lse: max|err| = {err:.3e}")
        assert err <= 1e-4 * max(1.0, float(np.abs(want_lse).max()))
        assert_close(down(o), oracle.causal_attention(f64(q, dtype), k64, v64, pos, shape.scale), TOL_BF16, "o")
        want = oracle.causal_attention_backward(f64(q, dtype), k64, v64, pos, shape.scale, f64(do, dtype))
        dq, dk, dv = _attn_bwd_run(torch, s, q, k, v, do, dtype, from_fwd=True)
        assert_close(dq, want["dq"], TOL_BF16, f"dq r={r}")
        assert_close(dk, want["dk"], TOL_BF16, f"dk r={r}")
        assert_close(dv, want["dv"], TOL_BF16, f"dv r={r}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attn_bwd_rank_contributions_sum(torch, dtype):
    """D emulated ranks over one sequence: each rank's dq rows are the
    full-sequence dq at its positions; the ranks' dK and dV add up to the
    full-sequence gradients."""
    S, D, H, Dh = 1024, 4, 2, 128 if dtype == "bf16" else 64
    shape = synth.LayerShape(S=S, D=D, h=H * Dh, H=H, Dh=Dh, F=256, dtype=dtype)
    k, v = synth.remote_kv(shape, seed=52)
    q_all = synth.normal((S, H, Dh), 52, synth.TID_Q, 0, dtype=dtype)
    do_all = synth.normal((S, H, Dh), 52, synth.TID_DY, 0, dtype=dtype)
    full = oracle.causal_attention_backward(f64(q_all, dtype), f64(k, dtype), f64(v, dtype), np.arange(S),
                                            shape.scale, f64(do_all, dtype))
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    dk_sum, dv_sum = np.zeros_like(full["dk"]), np.zeros_like(full["dv"])
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        s = tsp.make_shape(S, D, r, H * Dh, H, Dh, 256, dtype=dtype)
        log(f"attention backward, emulated rank {r} of {D}, {dtype}")
        dq, dk, dv = _attn_bwd_run(torch, s, q_all[pos], k, v, do_all[pos], dtype)
        assert_close(dq, full["dq"][pos], tol, f"dq rows of rank {r}")
        dk_sum += dk
        dv_sum += dv
    assert_close(dk_sum, full["dk"], tol, "sum of dK contributions")
    assert_close(dv_sum, full["dv"], tol, "sum of dV contributions")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("from_fwd", [False, True])
def test_attn_bwd_7b(torch, from_fwd):
    """7B attention (32 heads x 128, S = 131072, D = 8), rank 0: for one
    whole head, dq of every local row and dK, dV of every key row of the
    sequence (the rank's contribution, which covers the key blocks on both
    sides of the chunk boundaries and the keys past the rank's last position)
    against the oracle, which works per head; over all heads, sum_u dV_u =
    sum_t dO_t and sum_u dK_u = 0 for every head and feature (the softmax
    weights sum to one, the score gradients of a row to zero)."""
    SH = synth.SEVEN_B
    N, S, H, Dh = SH.N, SH.S, SH.H, SH.Dh
    r = 0
    q = synth.attn_queries(SH, seed=53)
    k, v = synth.remote_kv(SH, seed=53)
    do = synth.normal((N, H, Dh), 53, synth.TID_DY, 0, dtype="bf16")
    s = tsp.make_shape(S, SH.D, r, SH.h, H, Dh, SH.F, dtype="bf16")
    log(f"attention backward 7B, rank 0, statistics from the forward: {from_fwd}")
    dq, dk, dv = _attn_bwd_run(torch, s, q, k, v, do, "bf16", from_fwd)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    pos = oracle.zigzag_positions(S, SH.D, r)
    hd = 5
    sl = slice(hd, hd + 1)
    want = oracle.causal_attention_backward(f64(q[:, sl], "bf16"), f64(k[:, sl], "bf16"), f64(v[:, sl], "bf16"),
                                            pos, SH.scale, f64(do[:, sl], "bf16"))
    assert_close(dq[:, sl], want["dq"], TOL_BF16, f"dq of head {hd}, all {N} rows")
    assert_close(dk[:, sl], want["dk"], TOL_BF16, f"dK of head {hd}, all {S} keys")
    assert_close(dv[:, sl], want["dv"], TOL_BF16, f"dV of head {hd}, all {S} keys")
    do64 = f64(do, "bf16")
    assert_close(dv.sum(axis=0), do64.sum(axis=0), TOL_BF16, "sum over keys of dV vs sum over rows of dO")
    # sum_u dK_u = 0: held against the scale of one key row's gradient
    rms_row = float(np.sqrt(np.mean(dk ** 2)))
    err = float(np.abs(dk.sum(axis=0)).max())
    log(f"  sum over keys of dK: max {err:.3e} (dK rms {rms_row:.3e})")
    assert err <= TOL_BF16 * rms_row * np.sqrt(S)


# ---------------------------------------------------------------- plain bf16 P and dS
@pytest.mark.parametrize("S,D,H,Hkv,Dh,dtype", [c for c in ATTN_BWD_CASES if c[-1] == "bf16"])
@pytest.mark.parametrize("from_fwd", [False, True])
def test_attn_bwd_plain_pds_every_rank(torch, S, D, H, Hkv, Dh, dtype, from_fwd):
    """tsp_zigzag_attn_bwd_ex with TSP_ATTN_BWD_PLAIN_PDS (P and dS rounded
    once to bf16, as the layer backward takes them), statistics computed or
    from the forward, every rank: the norm-wise rule of the bf16 gradients
    against the oracle."""
    shape = synth.LayerShape(S=S, D=D, h=H * Dh, H=H, Dh=Dh, F=64 * D, dtype=dtype, Hkv=Hkv)
    N = S // D
    k, v = synth.remote_kv(shape, seed=51)
    for r in range(D):
        q = synth.normal((N, H, Dh), 51, synth.TID_Q, r, dtype=dtype)
        do = synth.normal((N, H, Dh), 51, synth.TID_DY, r, dtype=dtype)
        pos = oracle.zigzag_positions(S, D, r)
        want = oracle.causal_attention_backward(f64(q, dtype), f64(k, dtype), f64(v, dtype), pos, shape.scale,
                                                f64(do, dtype))
        s = tsp.make_shape(S, D, r, H * Dh, H, Dh, 64 * D, dtype=dtype, Hkv=Hkv)
        log(f"attention backward, plain P and dS, S={S} D={D} r={r} H={H} Hkv={Hkv} Dh={Dh} from_fwd={from_fwd}")
        dq, dk, dv = _attn_bwd_run(torch, s, q, k, v, do, dtype, from_fwd, tsp.TSP_ATTN_BWD_PLAIN_PDS)
        assert_close_nw(dq, want["dq"], f"dq r={r}")
        assert_close_nw(dk, want["dk"], f"dk r={r}")
        assert_close_nw(dv, want["dv"], f"dv r={r}")
        assert not dk[pos.max() + 1:].any() and not dv[pos.max() + 1:].any()


@pytest.mark.timeout(900)
def test_attn_bwd_plain_pds_7b(torch):
    """The 7B attention backward with plain bf16 P and dS and the forward's
    statistics (the layer backward's call), rank 0: dq of every local row and
    dK, dV of every key row for one whole head, norm-wise."""
    SH = synth.SEVEN_B
    N, S, H, Dh = SH.N, SH.S, SH.H, SH.Dh
    q = synth.attn_queries(SH, seed=53)
    k, v = synth.remote_kv(SH, seed=53)
    do = synth.normal((N, H, Dh), 53, synth.TID_DY, 0, dtype="bf16")
    s = tsp.make_shape(S, SH.D, 0, SH.h, H, Dh, SH.F, dtype="bf16")
    log("attention backward 7B, rank 0, plain P and dS, statistics from the forward")
    dq, dk, dv = _attn_bwd_run(torch, s, q, k, v, do, "bf16", True, tsp.TSP_ATTN_BWD_PLAIN_PDS)
    pos = oracle.zigzag_positions(S, SH.D, 0)
    hd = 5
    sl = slice(hd, hd + 1)
    want = oracle.causal_attention_backward(f64(q[:, sl], "bf16"), f64(k[:, sl], "bf16"), f64(v[:, sl], "bf16"),
                                            pos, SH.scale, f64(do[:, sl], "bf16"))
    assert_close_nw(dq[:, sl], want["dq"], f"dq of head {hd}, all {N} rows")
    assert_close_nw(dk[:, sl], want["dk"], f"dK of head {hd}, all {S} keys")
    assert_close_nw(dv[:, sl], want["dv"], f"dV of head {hd}, all {S} keys")
