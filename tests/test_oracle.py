"""Pins for the CPU oracle: each check comes from something other than the
oracle itself (hand-derived fixtures, textbook values, closed forms,
invariants, brute-force loops, or an independent library routine)."""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(t) for t in line.split()])
    return rows


# ---------------------------------------------------------------- zigzag
def test_zigzag_golden():
    for row in _load("zigzag_S16_D4.txt"):
        r = int(row[0])
        assert oracle.zigzag_positions(16, 4, r).tolist() == [int(t) for t in row[1:]]


@pytest.mark.parametrize("S,D", [(16, 4), (1024, 4), (64, 1), (96, 3), (4096, 8)])
def test_zigzag_permutation_and_equal_work(S, D):
    allpos = np.concatenate([oracle.zigzag_positions(S, D, r) for r in range(D)])
    assert sorted(allpos.tolist()) == list(range(S))
    # causal work of a rank = number of (query, key) pairs with key <= query
    work = [int((oracle.zigzag_positions(S, D, r) + 1).sum()) for r in range(D)]
    assert len(set(work)) == 1
    assert work[0] * D == S * (S + 1) // 2


def test_zigzag_d1_identity_and_owner():
    assert oracle.zigzag_positions(32, 1, 0).tolist() == list(range(32))
    S, D = 1024, 4
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        for t, p in enumerate(pos):
            assert oracle.zigzag_owner(int(p), S, D) == (r, t)


def test_zigzag_7b_pairs():
    S, D = 131072, 8
    for r in (0, 3, 7):
        assert int((oracle.zigzag_positions(S, D, r) + 1).sum()) == 1_073_750_016


def test_zigzag_rejects_bad_args():
    for S, D, r in [(10, 4, 0), (16, 4, 4), (16, 4, -1), (16, 0, 0)]:
        with pytest.raises(ValueError):
            oracle.zigzag_positions(S, D, r)


# ---------------------------------------------------------------- RMSNorm
def test_rms_norm_closed_forms():
    c, eps = 3.0, 1e-5
    x = np.full((2, 8), c)
    g = np.linspace(0.5, 2.0, 8)
    y = oracle.rms_norm(x, g, eps)
    assert np.allclose(y, c / math.sqrt(c * c + eps) * g, rtol=0, atol=1e-15)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    y = oracle.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-14)
    # scale invariance with eps = 0
    assert np.allclose(oracle.rms_norm(7.0 * x, np.ones(64), 0.0), y, atol=1e-14)


def test_rms_norm_vs_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 48))
    g = 1 + 0.1 * rng.standard_normal(48)
    ref = F.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(g), eps=1e-5).numpy()
    assert np.allclose(oracle.rms_norm(x, g, 1e-5), ref, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- GELU
def test_gelu_golden():
    for z, want in _load("gelu_values.txt"):
        assert abs(float(oracle.gelu(np.array([z]))[0]) - want) <= 1e-15 * max(1.0, abs(want))


def test_gelu_vs_math_erf_and_identities():
    zs = np.linspace(-6, 6, 97)
    got = oracle.gelu(zs)
    for z, gz in zip(zs, got):
        assert abs(gz - z * 0.5 * (1 + math.erf(z / math.sqrt(2)))) < 1e-15
    assert np.allclose(got - oracle.gelu(-zs), zs, atol=1e-14)  # x*Phi(x) - (-x)*Phi(-x) = x
    ref = F.gelu(torch.from_numpy(zs), approximate="none").numpy()
    assert np.allclose(got, ref, atol=1e-15)
    tanh_form = F.gelu(torch.from_numpy(zs), approximate="tanh").numpy()
    assert np.abs(got - tanh_form).max() > 1e-4  # the erf form is the one pinned


# ---------------------------------------------------------------- attention
def _brute_attention(q, k, v, q_pos, scale):
    n, H, Dh = q.shape
    out = np.zeros((n, H, Dh))
    for t in range(n):
        for hd in range(H):
            scores = []
            for u in range(int(q_pos[t]) + 1):
                scores.append(scale * sum(q[t, hd, d] * k[u, hd, d] for d in range(Dh)))
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            z = sum(w)
            for d in range(Dh):
                out[t, hd, d] = sum(w[u] * v[u, hd, d] for u in range(len(w))) / z
    return out


def test_attention_bruteforce_zigzag():
    rng = np.random.default_rng(2)
    S, D, H, Dh = 16, 2, 2, 3
    k = rng.standard_normal((S, H, Dh))
    v = rng.standard_normal((S, H, Dh))
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        q = rng.standard_normal((len(pos), H, Dh))
        got = oracle.causal_attention(q, k, v, pos, 0.7, row_block=3)
        assert np.allclose(got, _brute_attention(q, k, v, pos, 0.7), atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    S, H, Dh = 12, 3, 4
    q = rng.standard_normal((S, H, Dh))
    k = rng.standard_normal((S, H, Dh))
    v = rng.standard_normal((S, H, Dh))
    pos = np.arange(S)
    o = oracle.causal_attention(q, k, v, pos, 0.5)
    assert np.allclose(o[0], v[0], atol=1e-15)  # the first token sees only itself
    prefix_mean = np.cumsum(v, axis=0) / (pos + 1)[:, None, None]
    assert np.allclose(oracle.causal_attention(q, k, v, pos, 0.0), prefix_mean, atol=1e-14)
    k_same = np.broadcast_to(k[:1], k.shape)
    assert np.allclose(oracle.causal_attention(q, k_same, v, pos, 0.9), prefix_mean, atol=1e-14)


def test_attention_vs_torch_sdpa():
    rng = np.random.default_rng(4)
    S, H, Dh = 96, 4, 16
    q, k, v = (rng.standard_normal((S, H, Dh)) for _ in range(3))
    scale = 1 / math.sqrt(Dh)
    got = oracle.causal_attention(q, k, v, np.arange(S), scale, row_block=40)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2).contiguous()  # noqa: E731
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=scale)
    assert np.allclose(got, ref.permute(1, 0, 2).numpy(), atol=1e-13)


# ---------------------------------------------------------------- shards
def _split_attention(wq, wk, wv, wo, D, H, Dh, Hkv=None):
    """Shard layout of the library: head group j's Q rows (H/D heads), then
    its K and V rows (Hkv/D heads each); W_O columns of its query heads."""
    Hkv = H if Hkv is None else Hkv
    hd, kd = (H // D) * Dh, (Hkv // D) * Dh
    wqkv = [np.concatenate([wq[j * hd:(j + 1) * hd], wk[j * kd:(j + 1) * kd], wv[j * kd:(j + 1) * kd]]) for j in range(D)]
    wos = [wo[:, j * hd:(j + 1) * hd] for j in range(D)]
    return wqkv, wos


def _split_mlp(W1, W2, D):
    f = W1.shape[0] // D
    return [W1[j * f:(j + 1) * f] for j in range(D)], [W2[:, j * f:(j + 1) * f] for j in range(D)]


def test_mlp_vs_torch_and_shard_sum():
    rng = np.random.default_rng(5)
    n, h, Fw, D = 9, 16, 64, 4
    x = rng.standard_normal((n, h))
    W1 = 0.2 * rng.standard_normal((Fw, h))
    W2 = 0.2 * rng.standard_normal((h, Fw))
    w1, w2 = _split_mlp(W1, W2, D)
    got = oracle.mlp(x, w1, w2)
    tx = torch.from_numpy(x)
    ref = F.linear(F.gelu(F.linear(tx, torch.from_numpy(W1))), torch.from_numpy(W2)).numpy()
    assert np.allclose(got, ref, atol=1e-13)
    # no all-reduce needed: the shard contributions sum to the unsharded branch,
    # in any ring order
    for r in range(D):
        acc = np.zeros_like(got)
        for t in range(D):
            j = (r - t) % D
            acc += oracle.mlp_shard(x, w1[j], w2[j])
        assert np.allclose(acc, got, atol=1e-13)


def _torch_rope(t, base):
    """Rotary embedding written as complex multiplication: pair i of features
    (i, i + Dh/2) is the complex number a + ib, multiplied by
    exp(i * pos * base^(-2i/Dh)). t: [H, S, Dh], positions 0..S-1."""
    H, S, Dh = t.shape
    half = Dh // 2
    z = torch.complex(t[..., :half], t[..., half:])
    freq = base ** (-torch.arange(0, Dh, 2, dtype=torch.float64) / Dh)
    rot = torch.polar(torch.ones(S, half, dtype=torch.float64), torch.arange(S, dtype=torch.float64)[:, None] * freq)
    zr = z * rot[None]
    return torch.cat([zr.real, zr.imag], dim=-1)


def _torch_layer(x, wq, wk, wv, wo, W1, W2, g1, g2, H, Dh, eps, scale, rope_base=0.0, Wu=None):
    """torch fp64 layer; with Wu given, W1 is the gate matrix of a SwiGLU MLP."""
    tx = torch.from_numpy(x)
    S, h = x.shape
    a = F.rms_norm(tx, (h,), torch.from_numpy(g1), eps=eps)
    heads = lambda m: F.linear(a, torch.from_numpy(m)).reshape(S, H, Dh).permute(1, 0, 2).contiguous()  # noqa: E731
    q, k = heads(wq), heads(wk)
    if rope_base > 0:
        q, k = _torch_rope(q, rope_base), _torch_rope(k, rope_base)
    o = F.scaled_dot_product_attention(q, k, heads(wv), is_causal=True, scale=scale)
    h1 = tx + F.linear(o.permute(1, 0, 2).reshape(S, h), torch.from_numpy(wo))
    m = F.rms_norm(h1, (h,), torch.from_numpy(g2), eps=eps)
    if Wu is not None:
        hid = F.silu(F.linear(m, torch.from_numpy(W1))) * F.linear(m, torch.from_numpy(Wu))
    else:
        hid = F.gelu(F.linear(m, torch.from_numpy(W1)))
    return (h1 + F.linear(hid, torch.from_numpy(W2))).numpy()


def _tiny_layer(seed, S=64, D=4, H=4, Dh=8, Fw=128):
    rng = np.random.default_rng(seed)
    h = H * Dh
    mats = dict(
        wq=0.2 * rng.standard_normal((h, h)), wk=0.2 * rng.standard_normal((h, h)),
        wv=0.2 * rng.standard_normal((h, h)), wo=0.2 * rng.standard_normal((h, h)),
        W1=0.2 * rng.standard_normal((Fw, h)), W2=0.2 * rng.standard_normal((h, Fw)),
        g1=1 + 0.1 * rng.standard_normal(h), g2=1 + 0.1 * rng.standard_normal(h))
    wqkv, wos = _split_attention(mats["wq"], mats["wk"], mats["wv"], mats["wo"], D, H, Dh)
    w1, w2 = _split_mlp(mats["W1"], mats["W2"], D)
    w = dict(wqkv=wqkv, wo=wos, w1=w1, w2=w2, g_attn=mats["g1"], g_mlp=mats["g2"])
    x = rng.standard_normal((S, h))
    return x, w, mats


def test_layer_full_vs_torch():
    H, Dh, eps = 4, 8, 1e-5
    scale = 1 / math.sqrt(Dh)
    x, w, m = _tiny_layer(6, H=H, Dh=Dh)
    got = oracle.layer_full(x, w, H, Dh, eps, scale)["y"]
    ref = _torch_layer(x, m["wq"], m["wk"], m["wv"], m["wo"], m["W1"], m["W2"], m["g1"], m["g2"], H, Dh, eps, scale)
    assert np.allclose(got, ref, atol=1e-12)


def test_layer_rank_rows_equal_unsharded_layer():
    S, D, H, Dh, eps = 64, 4, 4, 8, 1e-5
    scale = 1 / math.sqrt(Dh)
    x, w, _ = _tiny_layer(7, S=S, D=D, H=H, Dh=Dh)
    full = oracle.layer_full(x, w, H, Dh, eps, scale)
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        # remote rows: garbage except what the all-gather would really carry
        k_remote = full["k"].copy()
        v_remote = full["v"].copy()
        k_remote[pos] = 1e3
        v_remote[pos] = -1e3
        out = oracle.layer_rank(x[pos], w, k_remote, v_remote, S, D, r, H, Dh, eps, scale)
        assert np.allclose(out["y"], full["y"][pos], atol=1e-12)
        sub = oracle.layer_rank(x[pos], w, k_remote, v_remote, S, D, r, H, Dh, eps, scale, rows=[0, 5, len(pos) - 1])
        assert np.allclose(sub["y"], full["y"][pos][[0, 5, len(pos) - 1]], atol=1e-12)


def test_layer_rank_d1_is_plain_layer():
    S, H, Dh, eps = 32, 2, 8, 1e-5
    x, w, _ = _tiny_layer(8, S=S, D=1, H=H, Dh=Dh, Fw=64)
    full = oracle.layer_full(x, w, H, Dh, eps, 0.3)
    junk = np.zeros((S, H, Dh))
    out = oracle.layer_rank(x, w, junk, junk, S, 1, 0, H, Dh, eps, 0.3)
    assert np.allclose(out["y"], full["y"], atol=1e-12)


# ---------------------------------------------------------------- rotary embedding (R7)
def test_rope_closed_forms():
    # one pair (Dh = 2): the angle is the position itself
    x = np.array([[[1.0, 0.0]], [[1.0, 0.0]], [[0.0, 2.0]]])
    got = oracle.rope(x, np.array([0, 1, 3]), 10000.0)
    want = np.array([[[1.0, 0.0]], [[math.cos(1), math.sin(1)]], [[-2 * math.sin(3), 2 * math.cos(3)]]])
    assert np.allclose(got, want, atol=1e-15)
    # Dh = 4, base 100: pair 1 turns at 1/10 of the position
    x = np.array([[[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]]])
    got = oracle.rope(x, np.array([5]), 100.0)
    assert np.allclose(got[0, 0], [math.cos(5), 0.0, math.sin(5), 0.0], atol=1e-15)
    assert np.allclose(got[0, 1], [0.0, math.cos(0.5), 0.0, math.sin(0.5)], atol=1e-15)
    # off, and position 0, leave x unchanged
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 2, 8))
    assert np.array_equal(oracle.rope(x, np.arange(3), 0.0), x)
    assert np.allclose(oracle.rope(x, np.zeros(3), 500.0), x, atol=0)


def test_rope_invariants():
    rng = np.random.default_rng(22)
    Dh, base = 16, 10000.0
    q, k = rng.standard_normal((2, 1, 1, Dh))
    # every pair keeps its length
    pos = np.array([12345])
    qr = oracle.rope(q, pos, base)[0, 0]
    assert np.allclose(qr[:8] ** 2 + qr[8:] ** 2, q[0, 0, :8] ** 2 + q[0, 0, 8:] ** 2, atol=1e-12)
    # scores depend on the position difference only
    for m, n, t in [(7, 3, 100), (0, 0, 131071), (50, 49, 5)]:
        a = np.dot(oracle.rope(q, [m], base).ravel(), oracle.rope(k, [n], base).ravel())
        b = np.dot(oracle.rope(q, [m + t], base).ravel(), oracle.rope(k, [n + t], base).ravel())
        assert abs(a - b) < 1e-10


def test_layer_with_rope_vs_torch_and_sharded():
    H, Dh, eps, base = 4, 8, 1e-5, 50.0
    scale = 1 / math.sqrt(Dh)
    S, D = 64, 4
    x, w, m = _tiny_layer(23, S=S, D=D, H=H, Dh=Dh)
    full = oracle.layer_full(x, w, H, Dh, eps, scale, rope_base=base)
    ref = _torch_layer(x, m["wq"], m["wk"], m["wv"], m["wo"], m["W1"], m["W2"], m["g1"], m["g2"], H, Dh, eps, scale,
                       rope_base=base)
    assert np.allclose(full["y"], ref, atol=1e-12)
    # the rank view reproduces its rows; remote K rows are the rotated ones
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        kr, vr = full["k"].copy(), full["v"].copy()
        kr[pos], vr[pos] = 1e3, -1e3
        out = oracle.layer_rank(x[pos], w, kr, vr, S, D, r, H, Dh, eps, scale, rope_base=base)
        assert np.allclose(out["y"], full["y"][pos], atol=1e-12)


# ---------------------------------------------------------------- grouped K/V heads (R8)
def test_gqa_attention_vs_torch():
    rng = np.random.default_rng(31)
    S, H, Hkv, Dh = 12, 6, 2, 4
    q = rng.standard_normal((S, H, Dh))
    k, v = rng.standard_normal((2, S, Hkv, Dh))
    got = oracle.causal_attention(q, k, v, np.arange(S), 0.7)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]  # noqa: E731  [1, heads, S, Dh]
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=0.7, enable_gqa=True)
    assert np.allclose(got, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


def _gqa_layer(seed, S, D, H, Hkv, Dh, Fw=96):
    rng = np.random.default_rng(seed)
    h, kvw = H * Dh, Hkv * Dh
    m = dict(wq=0.2 * rng.standard_normal((h, h)), wk=0.2 * rng.standard_normal((kvw, h)),
             wv=0.2 * rng.standard_normal((kvw, h)), wo=0.2 * rng.standard_normal((h, h)),
             W1=0.2 * rng.standard_normal((Fw, h)), W2=0.2 * rng.standard_normal((h, Fw)),
             g1=1 + 0.1 * rng.standard_normal(h), g2=1 + 0.1 * rng.standard_normal(h))
    w1, w2 = _split_mlp(m["W1"], m["W2"], D)
    return rng.standard_normal((S, h)), m, w1, w2


def test_gqa_layer_equals_mha_with_repeated_kv_heads():
    """A grouped layer equals the multi-head layer whose K/V weight rows are
    repeated for every query head of the group (an independent construction),
    for the unsharded layer and for every rank's view, with rotation too."""
    S, D, H, Hkv, Dh, eps, base = 32, 2, 4, 2, 8, 1e-5, 100.0
    scale = 1 / math.sqrt(Dh)
    x, m, w1, w2 = _gqa_layer(32, S, D, H, Hkv, Dh)
    g = H // Hkv
    rep = lambda wm: np.concatenate([np.repeat(wm[i * Dh:(i + 1) * Dh][None], g, 0).reshape(g * Dh, -1)  # noqa: E731
                                     for i in range(Hkv)])
    wqkv, wos = _split_attention(m["wq"], m["wk"], m["wv"], m["wo"], D, H, Dh, Hkv)
    wqkv_mha, wos_mha = _split_attention(m["wq"], rep(m["wk"]), rep(m["wv"]), m["wo"], D, H, Dh)
    w = dict(wqkv=wqkv, wo=wos, w1=w1, w2=w2, g_attn=m["g1"], g_mlp=m["g2"])
    w_mha = dict(wqkv=wqkv_mha, wo=wos_mha, w1=w1, w2=w2, g_attn=m["g1"], g_mlp=m["g2"])
    for rb in (0.0, base):
        full = oracle.layer_full(x, w, H, Dh, eps, scale, rope_base=rb, Hkv=Hkv)
        mha = oracle.layer_full(x, w_mha, H, Dh, eps, scale, rope_base=rb)
        assert full["k"].shape == (S, Hkv, Dh)
        assert np.allclose(full["y"], mha["y"], atol=1e-12)
        ref = _torch_layer(x, m["wq"], rep(m["wk"]), rep(m["wv"]), m["wo"], m["W1"], m["W2"], m["g1"], m["g2"], H, Dh,
                           eps, scale, rope_base=rb)
        assert np.allclose(full["y"], ref, atol=1e-12)
        for r in range(D):
            pos = oracle.zigzag_positions(S, D, r)
            kr, vr = full["k"].copy(), full["v"].copy()
            kr[pos], vr[pos] = 1e3, -1e3
            out = oracle.layer_rank(x[pos], w, kr, vr, S, D, r, H, Dh, eps, scale, rope_base=rb, Hkv=Hkv)
            assert np.allclose(out["y"], full["y"][pos], atol=1e-12)


# ---------------------------------------------------------------- planted mistakes
# ---------------------------------------------------------------- gated MLP (R9)
def test_silu_closed_forms_and_identities():
    # sigma(ln 3) = 1 / (1 + 1/3) = 3/4 and sigma(-ln 3) = 1/4, so SiLU there
    # is (3/4) ln 3 and -(1/4) ln 3; sigma(0) = 1/2 gives SiLU(0) = 0
    l3 = math.log(3.0)
    got = oracle.silu(np.array([0.0, l3, -l3]))
    assert np.allclose(got, [0.0, 0.75 * l3, -0.25 * l3], rtol=0, atol=1e-15)
    z = np.linspace(-30, 30, 241)
    # SiLU(z) - SiLU(-z) = z (sigma(z) + sigma(-z) = 1)
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, atol=1e-13)
    # far tails: z and 0, without overflow
    with np.errstate(all="raise"):
        big = oracle.silu(np.array([-800.0, 800.0]))
    assert big[0] == 0.0 and big[1] == 800.0
    assert np.allclose(oracle.silu(z), F.silu(torch.from_numpy(z)).numpy(), atol=1e-14)


def _split_gated(Wg, Wu, W2, D):
    """Shard j of a gated MLP: its W_g rows above its W_u rows (reading R9)."""
    f = Wg.shape[0] // D
    w1 = [np.concatenate([Wg[j * f:(j + 1) * f], Wu[j * f:(j + 1) * f]]) for j in range(D)]
    return w1, [W2[:, j * f:(j + 1) * f] for j in range(D)]


def test_gated_mlp_vs_torch_and_shard_sum():
    rng = np.random.default_rng(41)
    n, h, Fw, D = 9, 16, 64, 4
    x = rng.standard_normal((n, h))
    Wg, Wu = 0.3 * rng.standard_normal((2, Fw, h))
    W2 = 0.3 * rng.standard_normal((h, Fw))
    w1, w2 = _split_gated(Wg, Wu, W2, D)
    got = oracle.mlp(x, w1, w2, gated=True)
    tx = torch.from_numpy(x)
    ref = F.linear(F.silu(F.linear(tx, torch.from_numpy(Wg))) * F.linear(tx, torch.from_numpy(Wu)),
                   torch.from_numpy(W2)).numpy()
    assert np.allclose(got, ref, atol=1e-13)
    for r in range(D):
        acc = np.zeros_like(got)
        for t in range(D):
            j = (r - t) % D
            acc += oracle.mlp_shard(x, w1[j], w2[j], gated=True)
        assert np.allclose(acc, got, atol=1e-13)
    # the plain MLP on the same numbers is something else
    assert not np.allclose(oracle.mlp(x, [a[:Fw // D] for a in w1], w2), got, atol=1e-3)


def test_gated_layer_vs_torch_and_rank_views():
    """The gated layer against a torch fp64 layer at D = 1, and every rank's
    view against the unsharded layer, with rotation and grouped K/V too."""
    S, D, H, Dh, eps, Fw = 64, 4, 4, 8, 1e-5, 128
    scale = 1 / math.sqrt(Dh)
    x, w, m = _tiny_layer(43, S=S, D=D, H=H, Dh=Dh, Fw=Fw)
    rng = np.random.default_rng(44)
    Wu = 0.2 * rng.standard_normal((Fw, H * Dh))
    w1, _ = _split_gated(m["W1"], Wu, m["W2"], D)
    wg = dict(w, w1=w1)
    ref = _torch_layer(x, m["wq"], m["wk"], m["wv"], m["wo"], m["W1"], m["W2"], m["g1"], m["g2"], H, Dh, eps, scale,
                       Wu=Wu)
    full = oracle.layer_full(x, wg, H, Dh, eps, scale, gated=True)
    assert np.allclose(full["y"], ref, atol=1e-12)
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        out = oracle.layer_rank(x[pos], wg, full["k"], full["v"], S, D, r, H, Dh, eps, scale, gated=True)
        assert np.allclose(out["y"], full["y"][pos], atol=1e-12)
    # composed with rotation and 2 K/V heads (D = 2)
    D2, Hkv = 2, 2
    x2, m2, _, _ = _gqa_layer(45, S, D2, H, Hkv, Dh)
    Wg2, Wu2 = 0.2 * rng.standard_normal((2, 96, H * Dh))
    W22 = 0.2 * rng.standard_normal((H * Dh, 96))
    g1, g2 = _split_gated(Wg2, Wu2, W22, D2)
    wqkv, wos = _split_attention(m2["wq"], m2["wk"], m2["wv"], m2["wo"], D2, H, Dh, Hkv)
    wc = dict(wqkv=wqkv, wo=wos, w1=g1, w2=g2, g_attn=m2["g1"], g_mlp=m2["g2"])
    fc = oracle.layer_full(x2, wc, H, Dh, eps, scale, rope_base=50.0, Hkv=Hkv, gated=True)
    for r in range(D2):
        pos = oracle.zigzag_positions(S, D2, r)
        out = oracle.layer_rank(x2[pos], wc, fc["k"], fc["v"], S, D2, r, H, Dh, eps, scale, rope_base=50.0, Hkv=Hkv,
                                gated=True)
        assert np.allclose(out["y"], fc["y"][pos], atol=1e-12)


def test_planted_mistakes_are_caught(monkeypatch):
    """Each pin above fails when a plausible slip is planted in the oracle."""
    rng = np.random.default_rng(9)
    S, H, Dh = 10, 2, 3
    q, k, v = (rng.standard_normal((S, H, Dh)) for _ in range(3))
    pos = np.arange(S)
    good = _brute_attention(q, k, v, pos, 0.6)
    # exclusive instead of inclusive mask
    bad = oracle.causal_attention(q, k, v, pos - 1 + (pos == 0), 0.6)
    assert not np.allclose(bad, good, atol=1e-6)
    # transposed q/k roles inside a head (wrong operand)
    bad2 = oracle.causal_attention(k, q, v, pos, 0.6)
    assert not np.allclose(bad2, good, atol=1e-6)
    # a tanh GELU would miss the golden values
    z = np.array([r[0] for r in _load("gelu_values.txt")])
    want = np.array([r[1] for r in _load("gelu_values.txt")])
    tanh_gelu = 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    assert np.abs(tanh_gelu - want).max() > 1e-5
    # a K/V layout slip (K and V rows swapped within a shard) breaks the layer pin
    H2, Dh2, eps = 4, 8, 1e-5
    x, w, m = _tiny_layer(6, H=H2, Dh=Dh2)
    hd = (H2 // 4) * Dh2
    w_bad = dict(w)
    w_bad["wqkv"] = [np.concatenate([s[:hd], s[2 * hd:], s[hd:2 * hd]]) for s in w["wqkv"]]
    ref = _torch_layer(x, m["wq"], m["wk"], m["wv"], m["wo"], m["W1"], m["W2"], m["g1"], m["g2"], H2, Dh2, eps, 1 / math.sqrt(Dh2))
    assert not np.allclose(oracle.layer_full(x, w_bad, H2, Dh2, eps, 1 / math.sqrt(Dh2))["y"], ref, atol=1e-6)
    # rotary slips: interleaved pairs (2i, 2i+1), or the opposite turn, miss
    # the complex-number form
    t = rng.standard_normal((2, 5, 8))
    want = _torch_rope(torch.from_numpy(t), 30.0).numpy()
    x5 = t.transpose(1, 0, 2)  # [S, H, Dh]
    interleaved = np.empty_like(x5)
    perm = np.concatenate([np.arange(0, 8, 2), np.arange(1, 8, 2)])
    interleaved[..., perm] = oracle.rope(x5[..., perm], np.arange(5), 30.0)
    assert not np.allclose(interleaved.transpose(1, 0, 2), want, atol=1e-6)
    flipped = oracle.rope(x5, -np.arange(5), 30.0)
    assert not np.allclose(flipped.transpose(1, 0, 2), want, atol=1e-6)
    assert np.allclose(oracle.rope(x5, np.arange(5), 30.0).transpose(1, 0, 2), want, atol=1e-12)
    # grouping K/V heads round-robin (head i reads i % Hkv) misses torch's GQA
    qg = rng.standard_normal((6, 4, 3))
    kg, vg = rng.standard_normal((2, 6, 2, 3))
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]  # noqa: E731
    ref = F.scaled_dot_product_attention(t(qg), t(kg), t(vg), is_causal=True, scale=0.5, enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    rr = oracle.causal_attention(qg, np.tile(kg, (1, 2, 1)), np.tile(vg, (1, 2, 1)), np.arange(6), 0.5)
    assert not np.allclose(rr, ref, atol=1e-6)
    assert np.allclose(oracle.causal_attention(qg, kg, vg, np.arange(6), 0.5), ref, atol=1e-12)
    # gated MLP slips: gate and up halves swapped inside a shard, or a plain
    # sigmoid gate, miss torch's SwiGLU
    xs = rng.standard_normal((5, 8))
    Wg, Wu = rng.standard_normal((2, 16, 8))
    W2 = rng.standard_normal((8, 16))
    w1, w2 = _split_gated(Wg, Wu, W2, 2)
    tx = torch.from_numpy(xs)
    ref = F.linear(F.silu(F.linear(tx, torch.from_numpy(Wg))) * F.linear(tx, torch.from_numpy(Wu)),
                   torch.from_numpy(W2)).numpy()
    swapped = [np.concatenate([a[8:], a[:8]]) for a in w1]
    assert not np.allclose(oracle.mlp(xs, swapped, w2, gated=True), ref, atol=1e-6)
    monkeypatch.setattr(oracle.tsp_oracle, "silu", lambda z: 1 / (1 + np.exp(-np.asarray(z, dtype=np.float64))))
    assert not np.allclose(oracle.mlp(xs, w1, w2, gated=True), ref, atol=1e-6)


# ---------------------------------------------------------------- MLP backward
def test_gelu_grad_closed_forms_and_identities():
    # GELU'(0) = Phi(0) = 1/2; GELU(z) - GELU(-z) = z gives GELU'(z) + GELU'(-z) = 1
    assert oracle.gelu_grad(0.0) == pytest.approx(0.5, abs=1e-15)
    z = np.linspace(-6, 6, 241)
    assert np.allclose(oracle.gelu_grad(z) + oracle.gelu_grad(-z), 1.0, atol=1e-14)
    # GELU'(1) = Phi(1) + phi(1), from the textbook values Phi(1) = 0.841344746...
    # and phi(1) = exp(-1/2)/sqrt(2 pi) = 0.241970724...
    assert oracle.gelu_grad(1.0) == pytest.approx(0.8413447460685429 + 0.24197072451914337, abs=1e-14)
    # tails: 1 far right, 0 far left
    assert oracle.gelu_grad(40.0) == pytest.approx(1.0, abs=1e-15)
    assert abs(oracle.gelu_grad(-40.0)) < 1e-15
    # central differences of math.erf's GELU, and torch autograd fp64
    gelu = lambda t: 0.5 * t * (1 + math.erf(t / math.sqrt(2)))  # noqa: E731
    e = 1e-6
    for t in (-3.1, -0.7, 0.2, 1.3, 4.0):
        assert oracle.gelu_grad(t) == pytest.approx((gelu(t + e) - gelu(t - e)) / (2 * e), abs=1e-8)
    tz = torch.from_numpy(z.copy()).requires_grad_(True)
    F.gelu(tz).sum().backward()
    assert np.allclose(oracle.gelu_grad(z), tz.grad.numpy(), atol=1e-14)


def _torch_mlp_grads(x, W1, W2, dy):
    tx = torch.from_numpy(x).requires_grad_(True)
    t1 = torch.from_numpy(W1).requires_grad_(True)
    t2 = torch.from_numpy(W2).requires_grad_(True)
    y = F.linear(F.gelu(F.linear(tx, t1)), t2)
    (y * torch.from_numpy(dy)).sum().backward()
    return tx.grad.numpy(), t1.grad.numpy(), t2.grad.numpy()


def test_mlp_backward_vs_torch_autograd():
    rng = np.random.default_rng(11)
    n, h, Fw, D = 13, 16, 64, 4
    x = rng.standard_normal((n, h))
    W1, W2 = 0.3 * rng.standard_normal((Fw, h)), 0.3 * rng.standard_normal((h, Fw))
    dy = rng.standard_normal((n, h))
    w1, w2 = _split_mlp(W1, W2, D)
    got = oracle.mlp_backward(x, w1, w2, dy)
    gx, g1, g2 = _torch_mlp_grads(x, W1, W2, dy)
    assert np.allclose(got["dx"], gx, atol=1e-13)
    assert np.allclose(np.concatenate(got["dw1"], axis=0), g1, atol=1e-13)
    assert np.allclose(np.concatenate(got["dw2"], axis=1), g2, atol=1e-13)


def test_mlp_backward_finite_differences():
    """Central differences of L = sum(dy * y) with y from oracle.mlp (the
    forward, pinned on its own) in chosen entries of x, W1 and W2."""
    rng = np.random.default_rng(12)
    n, h, Fw, D = 5, 6, 8, 2
    x = rng.standard_normal((n, h))
    W1, W2 = 0.5 * rng.standard_normal((Fw, h)), 0.5 * rng.standard_normal((h, Fw))
    dy = rng.standard_normal((n, h))
    got = oracle.mlp_backward(x, *_split_mlp(W1, W2, D), dy)
    dW1, dW2 = np.concatenate(got["dw1"], axis=0), np.concatenate(got["dw2"], axis=1)
    loss = lambda x_, a, b: float((dy * oracle.mlp(x_, *_split_mlp(a, b, D))).sum())  # noqa: E731
    e = 1e-6
    for (i, j) in [(0, 0), (2, 5), (4, 3)]:
        xp, xm = x.copy(), x.copy()
        xp[i, j] += e
        xm[i, j] -= e
        assert got["dx"][i, j] == pytest.approx((loss(xp, W1, W2) - loss(xm, W1, W2)) / (2 * e), abs=1e-7)
    for (i, j) in [(0, 1), (5, 4), (7, 0)]:
        ap, am = W1.copy(), W1.copy()
        ap[i, j] += e
        am[i, j] -= e
        assert dW1[i, j] == pytest.approx((loss(x, ap, W2) - loss(x, am, W2)) / (2 * e), abs=1e-7)
    for (i, j) in [(0, 7), (3, 2), (5, 5)]:
        bp, bm = W2.copy(), W2.copy()
        bp[i, j] += e
        bm[i, j] -= e
        assert dW2[i, j] == pytest.approx((loss(x, W1, bp) - loss(x, W1, bm)) / (2 * e), abs=1e-7)


def test_mlp_backward_rank_contributions_sum_to_full_gradient():
    """Reading R10: every rank's rows of dx are the full-sequence dx at its
    positions, and the D ranks' weight-gradient contributions add up to the
    gradient over the whole sequence."""
    rng = np.random.default_rng(13)
    S, D, h, Fw = 32, 4, 8, 32
    x, dy = rng.standard_normal((2, S, h))
    W1, W2 = 0.3 * rng.standard_normal((Fw, h)), 0.3 * rng.standard_normal((h, Fw))
    w1, w2 = _split_mlp(W1, W2, D)
    full = oracle.mlp_backward(x, w1, w2, dy)
    acc1 = [np.zeros_like(a) for a in full["dw1"]]
    acc2 = [np.zeros_like(a) for a in full["dw2"]]
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        part = oracle.mlp_backward(x[pos], w1, w2, dy[pos])
        assert np.allclose(part["dx"], full["dx"][pos], atol=1e-13)
        for j in range(D):
            acc1[j] += part["dw1"][j]
            acc2[j] += part["dw2"][j]
    for j in range(D):
        assert np.allclose(acc1[j], full["dw1"][j], atol=1e-12)
        assert np.allclose(acc2[j], full["dw2"][j], atol=1e-12)


def test_mlp_backward_planted_mistakes_are_caught(monkeypatch):
    """GELU' without its z*phi(z) term, or the tanh form's derivative, misses
    torch's gradients."""
    rng = np.random.default_rng(14)
    n, h, Fw, D = 7, 8, 16, 2
    x = rng.standard_normal((n, h))
    W1, W2 = 0.5 * rng.standard_normal((Fw, h)), 0.5 * rng.standard_normal((h, Fw))
    dy = rng.standard_normal((n, h))
    gx, g1, _ = _torch_mlp_grads(x, W1, W2, dy)
    phi_only = lambda z: 0.5 * (1 + np.vectorize(math.erf)(np.asarray(z, dtype=np.float64) / math.sqrt(2)))  # noqa: E731
    monkeypatch.setattr(oracle.tsp_oracle, "gelu_grad", phi_only)
    bad = oracle.mlp_backward(x, *_split_mlp(W1, W2, D), dy)
    assert not np.allclose(bad["dx"], gx, atol=1e-6)
    assert not np.allclose(np.concatenate(bad["dw1"], axis=0), g1, atol=1e-6)


# ---------------------------------------------------------------- attention backward
def _torch_attn_grads(q, k, v, do, scale, gqa=False):
    """torch fp64 autograd through scaled_dot_product_attention (causal, all
    positions 0..S-1); q [S, H, Dh], k/v [S, Hkv, Dh]."""
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None].contiguous().requires_grad_(True)  # noqa: E731
    tq, tk, tv = t(q), t(k), t(v)
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale, enable_gqa=gqa)
    (o * torch.from_numpy(do).permute(1, 0, 2)[None]).sum().backward()
    back = lambda g: g[0].permute(1, 0, 2).numpy()  # noqa: E731
    return back(tq.grad), back(tk.grad), back(tv.grad)


@pytest.mark.parametrize("Hkv", [3, 1])
def test_attention_backward_vs_torch_autograd(Hkv):
    rng = np.random.default_rng(21)
    S, H, Dh, scale = 20, 3, 5, 0.4
    q = rng.standard_normal((S, H, Dh))
    k, v = rng.standard_normal((2, S, Hkv, Dh))
    do = rng.standard_normal((S, H, Dh))
    got = oracle.causal_attention_backward(q, k, v, np.arange(S), scale, do, row_block=7)
    gq, gk, gv = _torch_attn_grads(q, k, v, do, scale, gqa=Hkv != H)
    assert np.allclose(got["dq"], gq, atol=1e-12)
    assert np.allclose(got["dk"], gk, atol=1e-12)
    assert np.allclose(got["dv"], gv, atol=1e-12)


def test_attention_backward_finite_differences():
    """Central differences of L = sum(do * o), o from causal_attention (pinned
    on its own), in chosen entries of q, k and v; zigzag query positions."""
    rng = np.random.default_rng(22)
    S, D, r, H, Dh, scale = 16, 2, 1, 2, 3, 0.7
    pos = oracle.zigzag_positions(S, D, r)
    q = rng.standard_normal((len(pos), H, Dh))
    k, v = rng.standard_normal((2, S, H, Dh))
    do = rng.standard_normal((len(pos), H, Dh))
    got = oracle.causal_attention_backward(q, k, v, pos, scale, do)
    loss = lambda q_, k_, v_: float((do * oracle.causal_attention(q_, k_, v_, pos, scale)).sum())  # noqa: E731
    e = 1e-6
    for name, arr, idx in [("dq", q, (3, 1, 2)), ("dq", q, (7, 0, 0)), ("dk", k, (0, 1, 1)), ("dk", k, (13, 0, 2)),
                           ("dv", v, (2, 1, 0)), ("dv", v, (12, 0, 1))]:
        ap, am = arr.copy(), arr.copy()
        ap[idx] += e
        am[idx] -= e
        args_p = [ap if a is arr else a for a in (q, k, v)]
        args_m = [am if a is arr else a for a in (q, k, v)]
        fd = (loss(*args_p) - loss(*args_m)) / (2 * e)
        assert got[name][idx] == pytest.approx(fd, abs=1e-7), name
    # keys past every query of this rank get no gradient
    assert not got["dk"][pos.max() + 1:].any() and not got["dv"][pos.max() + 1:].any()


def test_attention_backward_rank_contributions_sum():
    """Reading R11: every rank's dq rows equal the full-sequence dq at its
    positions, and the ranks' dK/dV contributions add up to the full ones."""
    rng = np.random.default_rng(23)
    S, D, H, Dh, scale = 32, 4, 2, 4, 0.5
    q_all = rng.standard_normal((S, H, Dh))
    k, v = rng.standard_normal((2, S, H, Dh))
    do_all = rng.standard_normal((S, H, Dh))
    full = oracle.causal_attention_backward(q_all, k, v, np.arange(S), scale, do_all)
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        part = oracle.causal_attention_backward(q_all[pos], k, v, pos, scale, do_all[pos])
        assert np.allclose(part["dq"], full["dq"][pos], atol=1e-13)
        dk += part["dk"]
        dv += part["dv"]
    assert np.allclose(dk, full["dk"], atol=1e-12)
    assert np.allclose(dv, full["dv"], atol=1e-12)


def test_attention_backward_special_cases():
    """Scale 0: uniform weights over the prefix, so dv_u = sum over queries
    t >= u of do_t / (t + 1) and dq = 0 (closed forms); the query at position
    0 sees only key 0, so its dq is 0 and its do goes wholly to dv_0."""
    rng = np.random.default_rng(24)
    S, H, Dh = 9, 1, 3
    q, k, v, do = rng.standard_normal((4, S, H, Dh))
    got = oracle.causal_attention_backward(q, k, v, np.arange(S), 0.0, do)
    assert np.allclose(got["dq"], 0.0, atol=1e-15)
    for u in range(S):
        want = sum(do[t, 0] / (t + 1) for t in range(u, S))
        assert np.allclose(got["dv"][u, 0], want, atol=1e-13)
    one = oracle.causal_attention_backward(q[:1], k, v, np.array([0]), 0.9, do[:1])
    assert np.allclose(one["dq"], 0.0, atol=1e-15)
    assert np.allclose(one["dv"][0], do[0], atol=1e-15) and not one["dv"][1:].any()


def test_attention_lse_closed_forms_and_scipy():
    rng = np.random.default_rng(26)
    S, H, Dh = 11, 2, 3
    q, k = rng.standard_normal((2, S, H, Dh))
    # scale 0: every visible score is 0, so the log-sum-exp is log(pos + 1)
    got0 = oracle.causal_attention_lse(q, k, np.arange(S), 0.0)
    assert np.allclose(got0, np.log(np.arange(1, S + 1))[None, :], atol=1e-14)
    # scipy's logsumexp over each visible prefix; large scores do not overflow
    from scipy.special import logsumexp
    got = oracle.causal_attention_lse(q, k, np.arange(S), 40.0, row_block=4)
    for hd in range(H):
        for t in range(S):
            want = logsumexp(40.0 * (k[:t + 1, hd] @ q[t, hd]))
            assert got[hd, t] == pytest.approx(want, abs=1e-11)
    assert np.isfinite(got).all()
    # the forward's probabilities are exp(s - lse): each row sums to one
    p_row = np.exp(0.5 * (k[:6, 1] @ q[5, 1]) - oracle.causal_attention_lse(q, k, np.arange(S), 0.5)[1, 5])
    assert p_row.sum() == pytest.approx(1.0, abs=1e-14)


def test_attention_backward_planted_mistakes_are_caught(monkeypatch):
    """A softmax Jacobian without its row-sum term, or gradients taken with
    an exclusive mask, miss torch's autograd."""
    rng = np.random.default_rng(25)
    S, H, Dh, scale = 12, 2, 4, 0.6
    q, k, v, do = rng.standard_normal((4, S, H, Dh))
    gq, gk, gv = _torch_attn_grads(q, k, v, do, scale)
    bad_mask = oracle.causal_attention_backward(q[1:], k, v, np.arange(1, S) - 1, scale, do[1:])
    assert not np.allclose(bad_mask["dq"], gq[1:], atol=1e-6)
    # the identity sum_u p_u (dp_u - sum_w p_w dp_w) = 0 holds only with the term
    p = np.full((1, 4), 0.25)
    dp = np.array([[1.0, -2.0, 0.5, 3.0]])
    assert abs(oracle.softmax_backward(p, dp).sum()) < 1e-15
    monkeypatch.setattr(oracle.tsp_oracle, "softmax_backward", lambda p_, dp_: p_ * dp_)
    bad = oracle.causal_attention_backward(q, k, v, np.arange(S), scale, do)
    assert not np.allclose(bad["dq"], gq, atol=1e-6)
    assert not np.allclose(bad["dk"], gk, atol=1e-6)
    assert np.allclose(bad["dv"], gv, atol=1e-12)  # dv does not go through the Jacobian


# ---------------------------------------------------------------- synth
def test_synth_deterministic_and_bf16_rounding():
    a = synth.normal((3, 5), 1, 7)
    b = synth.normal((3, 5), 1, 7)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, synth.normal((3, 5), 1, 8))
    # RNE to bf16: ties go to even, widening is exact
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 65504.0], dtype=np.float32)
    bits = synth.f32_to_bf16(vals)
    back = synth.bf16_to_f32(bits)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 65536.0]
    big = synth.normal(((1 << 23) + 5,), 3, 1)  # several chunks
    assert np.array_equal(big[: 1 << 22], synth.normal((1 << 22,), 3, 1))  # chunked streams
    assert abs(float(big.mean())) < 2e-3 and abs(float(big.std()) - 1) < 2e-3


# ---------------------------------------------------------------- layer backward (R12)
def test_rms_norm_backward_vs_torch_autograd():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((6, 24))
    g = 1 + 0.2 * rng.standard_normal(24)
    dout = rng.standard_normal((6, 24))
    tx, tg = torch.from_numpy(x).requires_grad_(True), torch.from_numpy(g).requires_grad_(True)
    (F.rms_norm(tx, (24,), tg, eps=1e-5) * torch.from_numpy(dout)).sum().backward()
    dx, dg = oracle.rms_norm_backward(x, g, 1e-5, dout)
    assert np.allclose(dx, tx.grad.numpy(), atol=1e-13)
    assert np.allclose(dg, tg.grad.numpy(), atol=1e-13)
    # a constant row is a fixed point of the norm's direction: the gradient
    # along x itself vanishes when eps = 0 (scale invariance)
    xc = rng.standard_normal((1, 24))
    dxc, _ = oracle.rms_norm_backward(xc, np.ones(24), 0.0, xc)
    assert abs(float((dxc * xc).sum())) < 1e-12


def _torch_layer_grads(x, m, dy, H, Dh, eps, scale, Hkv):
    """torch fp64 autograd of the layer (grouped K/V heads as repeated heads
    inside scaled_dot_product_attention's enable_gqa)."""
    t = {k: torch.from_numpy(v).requires_grad_(True) for k, v in m.items()}
    tx = torch.from_numpy(x).requires_grad_(True)
    S, h = x.shape
    a = F.rms_norm(tx, (h,), t["g1"], eps=eps)
    heads = lambda w, nh: F.linear(a, w).reshape(S, nh, Dh).permute(1, 0, 2).contiguous()  # noqa: E731
    o = F.scaled_dot_product_attention(heads(t["wq"], H), heads(t["wk"], Hkv), heads(t["wv"], Hkv), is_causal=True,
                                       scale=scale, enable_gqa=Hkv != H)
    h1 = tx + F.linear(o.permute(1, 0, 2).reshape(S, h), t["wo"])
    mm = F.rms_norm(h1, (h,), t["g2"], eps=eps)
    y = h1 + F.linear(F.gelu(F.linear(mm, t["W1"])), t["W2"])
    (y * torch.from_numpy(dy)).sum().backward()
    return tx.grad.numpy(), {k: v.grad.numpy() for k, v in t.items()}


def _layer_bwd_case(seed, S=24, D=2, H=4, Hkv=4, Dh=4, Fw=32):
    rng = np.random.default_rng(seed)
    h = H * Dh
    m = dict(wq=0.3 * rng.standard_normal((h, h)), wk=0.3 * rng.standard_normal((Hkv * Dh, h)),
             wv=0.3 * rng.standard_normal((Hkv * Dh, h)), wo=0.3 * rng.standard_normal((h, h)),
             W1=0.3 * rng.standard_normal((Fw, h)), W2=0.3 * rng.standard_normal((h, Fw)),
             g1=1 + 0.1 * rng.standard_normal(h), g2=1 + 0.1 * rng.standard_normal(h))
    hq, hk = (H // D) * Dh, (Hkv // D) * Dh
    wqkv = [np.concatenate([m["wq"][j * hq:(j + 1) * hq], m["wk"][j * hk:(j + 1) * hk],
                            m["wv"][j * hk:(j + 1) * hk]], axis=0) for j in range(D)]
    wo = [m["wo"][:, j * hq:(j + 1) * hq] for j in range(D)]
    w1, w2 = _split_mlp(m["W1"], m["W2"], D)
    w = dict(wqkv=wqkv, wo=wo, w1=w1, w2=w2, g_attn=m["g1"], g_mlp=m["g2"])
    return rng.standard_normal((S, h)), rng.standard_normal((S, h)), w, m


@pytest.mark.parametrize("Hkv", [4, 2])
def test_layer_backward_vs_torch_autograd(Hkv):
    H, Dh, eps, scale = 4, 4, 1e-5, 0.5
    x, dy, w, m = _layer_bwd_case(32, Hkv=Hkv)
    got = oracle.layer_backward_full(x, w, dy, H, Dh, eps, scale, Hkv)
    gx, gm = _torch_layer_grads(x, m, dy, H, Dh, eps, scale, Hkv)
    assert np.allclose(got["dx"], gx, atol=1e-12)
    hq, hk = 2 * Dh, Hkv // 2 * Dh
    dwq = np.concatenate([d[:hq] for d in got["dwqkv"]], axis=0)
    dwk = np.concatenate([d[hq:hq + hk] for d in got["dwqkv"]], axis=0)
    dwv = np.concatenate([d[hq + hk:] for d in got["dwqkv"]], axis=0)
    for name, a in (("wq", dwq), ("wk", dwk), ("wv", dwv), ("wo", np.concatenate(got["dwo"], axis=1)),
                    ("W1", np.concatenate(got["dw1"], axis=0)), ("W2", np.concatenate(got["dw2"], axis=1)),
                    ("g1", got["dg_attn"]), ("g2", got["dg_mlp"])):
        assert np.allclose(a, gm[name], atol=1e-12), name


def test_layer_backward_finite_differences():
    """Central differences of L = sum(dy * y), y from oracle.layer_full (the
    forward, pinned on its own), in entries of x, the QKV and out-proj shards,
    W1 and both gains."""
    H, Dh, eps, scale = 4, 4, 1e-5, 0.5
    x, dy, w, _ = _layer_bwd_case(33, S=12)
    got = oracle.layer_backward_full(x, w, dy, H, Dh, eps, scale)

    def loss(x_, w_):
        return float((dy * oracle.layer_full(x_, w_, H, Dh, eps, scale)["y"]).sum())

    e = 1e-6

    def fd(path, idx):
        wp = {k: ([a.copy() for a in v] if isinstance(v, list) else v.copy()) for k, v in w.items()}
        wm = {k: ([a.copy() for a in v] if isinstance(v, list) else v.copy()) for k, v in w.items()}
        if path == "x":
            xp, xm = x.copy(), x.copy()
            xp[idx] += e
            xm[idx] -= e
            return (loss(xp, w) - loss(xm, w)) / (2 * e)
        key, j = path
        tp = wp[key][j] if j is not None else wp[key]
        tm = wm[key][j] if j is not None else wm[key]
        tp[idx] += e
        tm[idx] -= e
        return (loss(x, wp) - loss(x, wm)) / (2 * e)

    for idx in [(0, 0), (5, 7), (11, 15)]:
        assert got["dx"][idx] == pytest.approx(fd("x", idx), abs=1e-7)
    for j, idx in [(0, (0, 3)), (1, (9, 2)), (1, (23, 14))]:  # Q, K and V rows of the shards
        assert got["dwqkv"][j][idx] == pytest.approx(fd(("wqkv", j), idx), abs=1e-7)
    assert got["dwo"][1][(4, 5)] == pytest.approx(fd(("wo", 1), (4, 5)), abs=1e-7)
    assert got["dw1"][0][(3, 9)] == pytest.approx(fd(("w1", 0), (3, 9)), abs=1e-7)
    assert got["dg_attn"][6] == pytest.approx(fd(("g_attn", None), (6,)), abs=1e-7)
    assert got["dg_mlp"][10] == pytest.approx(fd(("g_mlp", None), (10,)), abs=1e-7)


@pytest.mark.parametrize("D,Hkv", [(4, 4), (2, 2)])
def test_layer_backward_rank_halves_compose(D, Hkv):
    """Reading R12 on D ranks: every rank runs the first half on its own rows
    (the gathered K/V of the full forward), the ranks' K/V gradients are
    summed and each rank takes the rows of its own positions into the second
    half. Every rank's dx rows are the full backward's at its positions, and
    the ranks' weight and gain contributions add up to the full gradients."""
    S, H, Dh, eps, scale = 32, 4, 4, 1e-5, 0.5
    x, dy, w, _ = _layer_bwd_case(34, S=S, D=D, Hkv=Hkv)
    full = oracle.layer_backward_full(x, w, dy, H, Dh, eps, scale, Hkv)
    fwd = oracle.layer_full(x, w, H, Dh, eps, scale, Hkv=Hkv)
    parts = [oracle.layer_bwd_attn_part(x[p], p, w, fwd["k"], fwd["v"], dy[p], H, Dh, eps, scale, Hkv)
             for p in (oracle.zigzag_positions(S, D, r) for r in range(D))]
    dk = sum(a["dk"] for a in parts)
    dv = sum(a["dv"] for a in parts)
    acc = {k: [np.zeros_like(t) for t in full[k]] for k in ("dwqkv", "dwo", "dw1", "dw2")}
    dg1, dg2 = np.zeros_like(full["dg_attn"]), np.zeros_like(full["dg_mlp"])
    for r, a in enumerate(parts):
        pos = oracle.zigzag_positions(S, D, r)
        b = oracle.layer_bwd_qkv_part(x[pos], w, a["dh1"], a["dq"], dk[pos], dv[pos], H, Dh, eps, Hkv)
        assert np.allclose(b["dx"], full["dx"][pos], atol=1e-12)
        for k, src in (("dwqkv", b), ("dwo", a), ("dw1", a), ("dw2", a)):
            for j in range(D):
                acc[k][j] += src[k][j]
        dg1 += b["dg_attn"]
        dg2 += a["dg_mlp"]
    for k in acc:
        for j in range(D):
            assert np.allclose(acc[k][j], full[k][j], atol=1e-12), k
    assert np.allclose(dg1, full["dg_attn"], atol=1e-12)
    assert np.allclose(dg2, full["dg_mlp"], atol=1e-12)


def test_layer_backward_planted_mistakes_are_caught(monkeypatch):
    """An RMSNorm backward without its mean term, or K and V gradients swapped
    in the QKV half, miss torch's gradients."""
    H, Dh, eps, scale = 4, 4, 1e-5, 0.5
    x, dy, w, m = _layer_bwd_case(35)
    gx, gm = _torch_layer_grads(x, m, dy, H, Dh, eps, scale, 4)
    good = oracle.rms_norm_backward

    def no_mean(x_, g_, eps_, dout):
        dx_, dg_ = good(x_, g_, eps_, dout)
        r = 1.0 / np.sqrt(np.mean(np.asarray(x_) ** 2, axis=-1, keepdims=True) + eps_)
        return r * np.asarray(g_) * np.asarray(dout), dg_

    monkeypatch.setattr(oracle.tsp_oracle, "rms_norm_backward", no_mean)
    assert not np.allclose(oracle.layer_backward_full(x, w, dy, H, Dh, eps, scale)["dx"], gx, atol=1e-6)
    monkeypatch.setattr(oracle.tsp_oracle, "rms_norm_backward", good)
    part = oracle.tsp_oracle.layer_bwd_qkv_part
    swapped = lambda x_, w_, dh1, dq, dk, dv, *a, **k: part(x_, w_, dh1, dq, dv, dk, *a, **k)  # noqa: E731
    monkeypatch.setattr(oracle.tsp_oracle, "layer_bwd_qkv_part", swapped)
    bad = oracle.tsp_oracle.layer_backward_full(x, w, dy, H, Dh, eps, scale)
    assert not np.allclose(bad["dx"], gx, atol=1e-6)
