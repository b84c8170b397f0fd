"""GPU parity of the layer backward (tsp_layer_bwd) against the fp64 oracle.

Small shapes, every rank: each rank runs the first half (TSP_BWD_ATTN) on
its own tokens; the D ranks' K/V-row gradients are summed and each rank's own
rows handed back (the reduce-scatter, emulated with a plain sum on the
device); each rank then runs the second half (TSP_BWD_QKV). Every output of
every rank is held against the oracle's two halves on the same inputs, and
the ranks' results together against the unsharded layer's backward. K/V are
the layer's own, computed by the oracle from the whole sequence and rounded
to the storage type.

7B (S=131072, D=8): the output gradient dy is zero outside a sample of rows
T, and so are the K/V-row gradients given to the second half. Every
gradient is then a sum over T alone (a zero dy row contributes nothing to
any weight, gain or K/V gradient, and its dx row is exactly zero), so the
oracle evaluates the two halves on the rows of T only and every output
element of the full-size call is compared.
"""
import numpy as np
import pytest

import oracle
import synth
import tsp_rank_local_amd as tsp
from gpu_util import TOL_F32, assert_close, assert_close_nw, down, f64, log, torch_cuda, up

pytestmark = pytest.mark.gpu

GRAD_KEYS = ("wqkv", "wo", "w1", "w2")


@pytest.fixture(scope="module")
def torch():
    t = torch_cuda()
    tsp.lib()
    return t


def _dev_weights(w, dtype):
    return {k: ([up(a, dtype) for a in w[k]] if isinstance(w[k], list) else up(w[k], dtype))
            for k in ("wqkv", "wo", "w1", "w2", "g_attn", "g_mlp")}


def _w64(w, dtype):
    return {k: ([f64(a, dtype) for a in w[k]] if isinstance(w[k], list) else f64(w[k], dtype)) for k in w}


def _grads(torch, w):
    """NaN-filled fp32 gradient buffers shaped like the weights (every element must be written)."""
    g = {k: [torch.full(a.shape, float("nan"), dtype=torch.float32, device="cuda") for a in w[k]] for k in GRAD_KEYS}
    for k in ("g_attn", "g_mlp"):
        g[k] = torch.full(w[k].shape, float("nan"), dtype=torch.float32, device="cuda")
    return g


def _nan(torch, *shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _true_kv(shape, w64, x_all):
    """The layer's K/V over the whole sequence (oracle, fp64), rounded to the storage type."""
    _, wk, wv, _ = oracle.unshard_attention_weights(w64["wqkv"], w64["wo"], shape.H, shape.Dh, shape.kv_heads)
    xn = oracle.rms_norm(x_all, w64["g_attn"], shape.eps)
    out = []
    for wm in (wk, wv):
        t = (xn @ wm.T).reshape(shape.S, shape.kv_heads, shape.Dh).astype(np.float32)
        out.append(synth.f32_to_bf16(t) if shape.dtype == "bf16" else t)
    return out


def _close(got, want, dtype, what):
    """fp32: max |err| <= 1e-4 rms; bf16: the norm-wise rule of the backward."""
    if dtype == "f32":
        assert_close(got, want, TOL_F32, what)
    else:
        assert_close_nw(got, want, what)


def _close_grads(got, want, dtype, tag, keys):
    """got: gradient buffers by weight name; want: the oracle's dict (keys 'd' + name)."""
    for k in keys:
        if k in ("g_attn", "g_mlp"):
            _close(down(got[k]), want["d" + k], dtype, f"d{k} {tag}")
        else:
            ax = 1 if k in ("wo", "w2") else 0
            _close(np.concatenate([down(a) for a in got[k]], axis=ax), np.concatenate(want["d" + k], axis=ax), dtype,
                   f"d{k} {tag}")


LAYER_BWD_CASES = [
    # S, D, h, H, Dh, F, Hkv, dtype
    (1024, 4, 256, 4, 64, 1024, 0, "f32"),     # the tiny fp32 layer
    (1024, 4, 256, 4, 64, 1024, 0, "bf16"),    # the same in bf16
    (1280, 2, 384, 6, 64, 768, 0, "bf16"),     # 640 tokens, h = 384, F/D = 384: ragged tiles everywhere
    (2048, 2, 512, 8, 64, 1024, 2, "bf16"),    # grouped K/V: one K/V head per shard
    (2048, 4, 512, 4, 128, 2048, 0, "bf16"),   # 128-wide heads
    (576, 3, 192, 3, 64, 192, 0, "bf16"),      # 192 tokens, h = F = 192: 3 K steps in every product, a new shard
                                               # every step in the ring-order ones, 96-row chunks
]


def _saved_forward(torch, s, wd, x, kd, vd, keep_z):
    """tsp_layer_fwd_save on the given K/V: PHASE_KV on scratch copies (the
    rank's own rows stay the given ones in kd, vd), then PHASE_REST on kd,
    vd with the same workspace. Returns the kept O, log-sum-exp and (keep_z)
    MLP pre-activation."""
    N, H, Dh = s.S // s.D, s.H, s.Dh
    ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")
    y = _nan(torch, N, s.h)
    o = _nan(torch, N, H, Dh)
    lse = _nan(torch, H, N)
    z = torch.full((N, s.F), float("nan"), dtype=torch.bfloat16, device="cuda") if keep_z else None
    tsp.tsp_layer_fwd_save(s, wd, x, kd.clone(), vd.clone(), y, o, lse, tsp.TSP_PHASE_KV, ws, z_save=z)
    tsp.tsp_layer_fwd_save(s, wd, x, kd, vd, y, o, lse, tsp.TSP_PHASE_REST, ws, z_save=z)
    return o, lse, z


@pytest.mark.parametrize("S,D,h,H,Dh,F,Hkv,dtype", LAYER_BWD_CASES)
def test_layer_bwd_every_rank(torch, S, D, h, H, Dh, F, Hkv, dtype):
    _layer_bwd_every_rank(torch, S, D, h, H, Dh, F, Hkv, dtype, saved=False)


@pytest.mark.parametrize("S,D,h,H,Dh,F,Hkv,dtype,keep_z",
                         [c + (True,) for c in LAYER_BWD_CASES if c[-1] == "bf16"] +
                         [LAYER_BWD_CASES[1] + (False,)])
def test_layer_bwd_saved_every_rank(torch, S, D, h, H, Dh, F, Hkv, dtype, keep_z):
    """tsp_layer_bwd_ex with the attention output and statistics (and the
    MLP pre-activation, keep_z) that tsp_layer_fwd_save kept, held to the same
    oracle and tolerances."""
    _layer_bwd_every_rank(torch, S, D, h, H, Dh, F, Hkv, dtype, saved=True, keep_z=keep_z)


def _layer_bwd_every_rank(torch, S, D, h, H, Dh, F, Hkv, dtype, saved, keep_z=False):
    shape = synth.LayerShape(S=S, D=D, h=h, H=H, Dh=Dh, F=F, dtype=dtype, Hkv=Hkv)
    N, Hk = S // D, shape.kv_heads
    w = synth.layer_weights(shape, seed=61, gain="random")
    w64, wd = _w64(w, dtype), _dev_weights(w, dtype)
    x_all = synth.activations(S, h, seed=61)                      # global order
    dy_all = synth.activations(S, h, seed=61, tid=synth.TID_DY)
    kf, vf = _true_kv(shape, w64, x_all)
    kf64, vf64 = f64(kf, dtype), f64(vf, dtype)
    kd, vd = up(kf, dtype), up(vf, dtype)
    pos = [oracle.zigzag_positions(S, D, r) for r in range(D)]
    shapes = [tsp.make_shape(S, D, r, h, H, Dh, F, eps=shape.eps, dtype=dtype, Hkv=Hkv) for r in range(D)]
    wss = [torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER_BWD), dtype=torch.uint8, device="cuda") for s in shapes]

    # first half on every rank
    xs = [up(np.ascontiguousarray(x_all[p]), "f32") for p in pos]
    dys = [up(np.ascontiguousarray(dy_all[p]), "f32") for p in pos]
    dkf = [_nan(torch, S, Hk, Dh) for _ in range(D)]
    dvf = [_nan(torch, S, Hk, Dh) for _ in range(D)]
    g = [_grads(torch, wd) for _ in range(D)]
    for r in range(D):
        log(f"layer bwd ATTN S={S} D={D} r={r} h={h} H={H} Hkv={Hk} Dh={Dh} F={F} {dtype}"
            f"{' from the saved forward' if saved else ''}")
        ga = {**g[r], "wqkv": None, "g_attn": None}
        if saved:
            o, lse, z = _saved_forward(torch, shapes[r], wd, xs[r], kd, vd, keep_z)
            tsp.tsp_layer_bwd_ex(shapes[r], wd, xs[r], kd, vd, dys[r], o, lse, dkf[r], dvf[r], None, None, None, ga,
                                 tsp.TSP_BWD_ATTN, wss[r], z_saved=z)
        else:
            tsp.tsp_layer_bwd(shapes[r], wd, xs[r], kd, vd, dys[r], dkf[r], dvf[r], None, None, None, ga,
                              tsp.TSP_BWD_ATTN, wss[r])
    torch.cuda.synchronize()
    a = [oracle.layer_bwd_attn_part(x_all[pos[r]], pos[r], w64, kf64, vf64, dy_all[pos[r]], H, Dh, shape.eps,
                                    shape.scale, Hk) for r in range(D)]
    for r in range(D):
        _close(down(dkf[r]), a[r]["dk"], dtype, f"dk_full r={r}")
        _close(down(dvf[r]), a[r]["dv"], dtype, f"dv_full r={r}")
        _close_grads(g[r], a[r], dtype, f"r={r}", ("wo", "w1", "w2", "g_mlp"))

    # the reduce-scatter: every rank gets the sum over ranks of its own rows
    dk_sum, dv_sum = sum(dkf[1:], dkf[0].clone()), sum(dvf[1:], dvf[0].clone())
    dk64, dv64 = sum(x["dk"] for x in a), sum(x["dv"] for x in a)
    dxs = [_nan(torch, N, h) for _ in range(D)]
    for r in range(D):
        p = torch.from_numpy(pos[r]).cuda()
        log(f"layer bwd QKV r={r}")
        tsp.tsp_layer_bwd(shapes[r], wd, xs[r], None, None, None, None, None, dk_sum[p].contiguous(),
                          dv_sum[p].contiguous(), dxs[r], {**g[r], "wo": None, "w1": None, "w2": None, "g_mlp": None},
                          tsp.TSP_BWD_QKV, wss[r])
    torch.cuda.synchronize()
    for r in range(D):
        b = oracle.layer_bwd_qkv_part(x_all[pos[r]], w64, a[r]["dh1"], a[r]["dq"], dk64[pos[r]], dv64[pos[r]], H,
                                      Dh, shape.eps, Hk)
        _close(down(dxs[r]), b["dx"], dtype, f"dx r={r}")
        _close_grads(g[r], b, dtype, f"r={r}", ("wqkv", "g_attn"))

    # the ranks together: the unsharded layer's backward over the sequence
    full = oracle.layer_backward_full(x_all, w64, dy_all, H, Dh, shape.eps, shape.scale, Hk)
    dx_all = np.empty((S, h))
    for r in range(D):
        dx_all[pos[r]] = down(dxs[r])
    _close(dx_all, full["dx"], dtype, "dx, all ranks")
    tot = {k: [sum(down(g[r][k][j]) for r in range(D)) for j in range(D)] for k in GRAD_KEYS}
    for k in ("g_attn", "g_mlp"):
        tot[k] = sum(down(g[r][k]) for r in range(D))
    for k in GRAD_KEYS:
        ax = 1 if k in ("wo", "w2") else 0
        _close(np.concatenate(tot[k], axis=ax), np.concatenate(full["d" + k], axis=ax), dtype,
               f"d{k} summed over ranks")
    for k in ("g_attn", "g_mlp"):
        _close(tot[k], full["d" + k], dtype, f"d{k} summed over ranks")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_bwd_one_rank_both_phases(torch, dtype):
    """D = 1: the rank owns every K/V row, so one TSP_BWD_ALL call with dk_loc
    = dk_full (and dv_loc = dv_full) is the whole layer's backward; run twice
    for bitwise determinism."""
    S, h, H, Dh, F = 512, 256, 2, 128, 512
    shape = synth.LayerShape(S=S, D=1, h=h, H=H, Dh=Dh, F=F, dtype=dtype)
    w = synth.layer_weights(shape, seed=62, gain="random")
    w64, wd = _w64(w, dtype), _dev_weights(w, dtype)
    x = synth.activations(S, h, seed=62)
    dy = synth.activations(S, h, seed=62, tid=synth.TID_DY)
    kf, vf = _true_kv(shape, w64, x)
    s = tsp.make_shape(S, 1, 0, h, H, Dh, F, eps=shape.eps, dtype=dtype)
    outs = []
    for it in range(2):
        ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER_BWD), dtype=torch.uint8, device="cuda")
        dk, dv, dx = _nan(torch, S, H, Dh), _nan(torch, S, H, Dh), _nan(torch, S, h)
        g = _grads(torch, wd)
        log(f"layer bwd D=1 ALL S={S} {dtype} run {it}")
        tsp.tsp_layer_bwd(s, wd, up(x, "f32"), up(kf, dtype), up(vf, dtype), up(dy, "f32"), dk, dv, dk, dv, dx, g,
                          tsp.TSP_BWD_ALL, ws)
        torch.cuda.synchronize()
        outs.append((down(dx), {k: [down(t) for t in g[k]] for k in GRAD_KEYS},
                     {k: down(g[k]) for k in ("g_attn", "g_mlp")}, down(dk)))
    dx0, gw0, gg0, dk0 = outs[0]
    dx1, gw1, gg1, dk1 = outs[1]
    assert np.array_equal(dx0, dx1) and np.array_equal(dk0, dk1)
    for k in GRAD_KEYS:
        assert all(np.array_equal(p, q) for p, q in zip(gw0[k], gw1[k])), k
    for k in gg0:
        assert np.array_equal(gg0[k], gg1[k]), k
    full = oracle.layer_backward_full(x, w64, dy, H, Dh, shape.eps, shape.scale)
    _close(dx0, full["dx"], dtype, "dx")
    for k in GRAD_KEYS:
        _close(np.concatenate(gw0[k], axis=1 if k in ("wo", "w2") else 0),
               np.concatenate(full["d" + k], axis=1 if k in ("wo", "w2") else 0), dtype, f"d{k}")
    for k in gg0:
        _close(gg0[k], full["d" + k], dtype, f"d{k}")


def _sample_rows(N, C):
    """Local rows of the 7B check: the first rows (rank 0's earliest
    positions), rows inside and at the end of the first chunk, the start of
    the second chunk and the last rows."""
    t = [0, 1, 2, 5, 63, 64, 1000, C - 1, C, C + 1, C + 4097, N - 3, N - 2, N - 1]
    return np.array(sorted(set(t)), dtype=np.int64)


@pytest.mark.parametrize("r,saved", [(0, False), (5, False), (0, True)])
def test_layer_bwd_7b_sampled_rows(torch, r, saved):
    """saved: the first half takes the attention output, statistics and MLP
    pre-activation of tsp_layer_fwd_save instead of running the attention
    forward and the MLP up product again."""
    shape = synth.SEVEN_B
    S, D, h, H, Dh, F = shape.S, shape.D, shape.h, shape.H, shape.Dh, shape.F
    N, C = S // D, S // (2 * D)
    T = _sample_rows(N, C)
    w = synth.layer_weights(shape, seed=63)
    wd = _dev_weights(w, "bf16")
    k_rem, v_rem = synth.remote_kv(shape, seed=63)
    x = synth.activations(N, h, seed=63, tid=100 + r)
    dy = np.zeros((N, h), dtype=np.float32)
    dy[T] = synth.activations(N, h, seed=63, tid=synth.TID_DY)[T]
    dkl = np.zeros((N, H, Dh), dtype=np.float32)
    dvl = np.zeros((N, H, Dh), dtype=np.float32)
    dkl[T] = synth.normal((N, H, Dh), 63, synth.TID_DK_LOC, std=0.05)[T]
    dvl[T] = synth.normal((N, H, Dh), 63, synth.TID_DV_LOC, std=0.05)[T]
    s = tsp.make_shape(S, D, r, h, H, Dh, F, eps=shape.eps, dtype="bf16")
    ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER_BWD), dtype=torch.uint8, device="cuda")
    dkf, dvf, dx = _nan(torch, S, H, Dh), _nan(torch, S, H, Dh), _nan(torch, N, h)
    g = _grads(torch, wd)
    log(f"layer bwd 7B S={S} D={D} r={r}: both phases, {len(T)} rows of dy{' from the saved forward' if saved else ''}")
    xd = up(x, "f32")
    kd, vd = up(k_rem, "bf16"), up(v_rem, "bf16")
    o, lse, z = _saved_forward(torch, s, wd, xd, kd, vd, True) if saved else (None, None, None)
    tsp.tsp_layer_bwd_ex(s, wd, xd, kd, vd, up(dy, "f32"), o, lse, dkf, dvf, None, None, None,
                         {**g, "wqkv": None, "g_attn": None}, tsp.TSP_BWD_ATTN, ws, z_saved=z)
    del o, lse, z, kd, vd
    tsp.tsp_layer_bwd(s, wd, xd, None, None, None, None, None, up(dkl, "f32"), up(dvl, "f32"), dx,
                      {**g, "wo": None, "w1": None, "w2": None, "g_mlp": None}, tsp.TSP_BWD_QKV, ws)
    torch.cuda.synchronize()
    del ws
    w64 = _w64(w, "bf16")
    pos = oracle.zigzag_positions(S, D, r)
    a = oracle.layer_bwd_attn_part(x[T], pos[T], w64, f64(k_rem, "bf16"), f64(v_rem, "bf16"), dy[T], H, Dh,
                                   shape.eps, shape.scale)
    b = oracle.layer_bwd_qkv_part(x[T], w64, a["dh1"], a["dq"], dkl[T], dvl[T], H, Dh, shape.eps)
    dx_got = down(dx)
    rest = np.ones(N, dtype=bool)
    rest[T] = False
    assert not np.any(dx_got[rest]), "dx rows outside the sample must be exactly zero"
    assert_close_nw(dx_got[T], b["dx"], f"dx rows r={r}")
    # K/V-row gradients: only keys at or before the sampled queries' positions
    lim = int(pos[T].max()) + 1
    dk_got, dv_got = down(dkf), down(dvf)
    assert not np.any(dk_got[lim:]) and not np.any(dv_got[lim:])
    assert_close_nw(dk_got[:lim], a["dk"][:lim], f"dk_full r={r}")
    assert_close_nw(dv_got[:lim], a["dv"][:lim], f"dv_full r={r}")
    _close_grads(g, {**a, **b}, "bf16", f"r={r}",
                 ("wqkv", "wo", "w1", "w2", "g_attn", "g_mlp"))


@pytest.mark.parametrize("S,D,h,H,Dh,F,Hkv", [(1024, 4, 256, 4, 64, 1024, 0), (2048, 2, 512, 8, 64, 1024, 2),
                                              (2048, 4, 512, 4, 128, 2048, 0)])
def test_layer_fwd_save_every_rank(torch, S, D, h, H, Dh, F, Hkv):
    """tsp_layer_fwd_save: y and the rank's K/V rows bit for bit those of
    tsp_layer_fwd; the kept O against the oracle's attention output (the
    backward's norm-wise rule), the kept log-sum-exp against the oracle's
    within the bf16 rounding of the scores."""
    shape = synth.LayerShape(S=S, D=D, h=h, H=H, Dh=Dh, F=F, dtype="bf16", Hkv=Hkv)
    N, Hk = S // D, shape.kv_heads
    w = synth.layer_weights(shape, seed=63, gain="random")
    w64, wd = _w64(w, "bf16"), _dev_weights(w, "bf16")
    k_rem, v_rem = synth.remote_kv(shape, seed=63)
    wq = oracle.unshard_attention_weights(w64["wqkv"], w64["wo"], H, Dh, Hk)[0]
    for r in range(D):
        x = synth.activations(N, h, seed=63 + r)
        s = tsp.make_shape(S, D, r, h, H, Dh, F, eps=shape.eps, dtype="bf16", Hkv=Hkv)
        log(f"layer fwd with the attention output kept: S={S} D={D} r={r} h={h} H={H} Hkv={Hk} Dh={Dh} F={F}")
        xd = up(x, "f32")
        ys, ks, vs = [], [], []
        o, lse = _nan(torch, N, H, Dh), _nan(torch, H, N)
        for save in (False, True):
            kd, vd = up(k_rem, "bf16"), up(v_rem, "bf16")
            ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")
            y = _nan(torch, N, h)
            if save:
                tsp.tsp_layer_fwd_save(s, wd, xd, kd, vd, y, o, lse, tsp.TSP_PHASE_ALL, ws)
            else:
                tsp.tsp_layer_fwd(s, wd, xd, kd, vd, y, tsp.TSP_PHASE_ALL, ws)
            torch.cuda.synchronize()
            ys.append(down(y))
            ks.append(down(kd))
            vs.append(down(vd))
        assert np.array_equal(ys[0], ys[1]), "y differs from tsp_layer_fwd"
        assert np.array_equal(ks[0], ks[1]) and np.array_equal(vs[0], vs[1])
        pos = oracle.zigzag_positions(S, D, r)
        k_all, v_all = f64(k_rem, "bf16").copy(), f64(v_rem, "bf16").copy()
        k_all[pos], v_all[pos] = oracle.local_kv(x, w64, H, Dh, shape.eps, pos, 0.0, Hk)
        q = (oracle.rms_norm(x, w64["g_attn"], shape.eps) @ wq.T).reshape(N, H, Dh)
        # O is an intermediate of bf16 Q, K and V (rounded once each): rows
        # that see few keys carry their rounding unaveraged (rank 0's first
        # rows near 2e-2 of the tensor's rms, and the forward recomputes
        # their y in fp32, not their kept O). The backward consumes O, so it
        # is held to the backward's norm-wise rule; y itself is bit for bit
        # that of tsp_layer_fwd, whose parity the forward tests hold.
        assert_close_nw(down(o), oracle.causal_attention(q, k_all, v_all, pos, shape.scale), f"o r={r}")
        want = oracle.causal_attention_lse(q, k_all, pos, shape.scale)
        got = down(lse)
        assert np.all(np.isfinite(got))
        # each score carries the bf16 rounding of its q and k (and of the
        # normed input behind q), at most about 2^-8 |q| |k| scale; the row's
        # log-sum-exp moves by at most its largest such change (bound taken
        # with a factor 2 to spare and the largest key norm of the head)
        qn = np.linalg.norm(q, axis=2)                                     # [N, H]
        kn = np.linalg.norm(k_all, axis=2).max(axis=0)                     # [Hkv]
        kn = np.repeat(kn, H // Hk)                                        # per query head
        tol = 2.0 ** -7 * shape.scale * (qn * kn[None, :]).T + 1e-4        # [H, N]
        err = np.abs(got - want)
        log(f"  lse: max|err| = {err.max():.3e}, worst err/bound = {(err / tol).max():.3f}")
        assert np.all(err <= tol), "log-sum-exp outside the rounding bound"

