"""Host checks of the analytic per-rank memory model: its workspace sizes
equal what the library asks for (tsp_workspace_size) on every kind of call
and variant, and its components follow what the zubnet.ai page states about
the folded axis (paragraph 1: weights and activations both fall as 1/D;
paragraph 2: the all-gather delivers the other ranks' K/V rows). No GPU."""
import itertools

import pytest

import tsp_rank_local_amd as tsp
from tsp_rank_local_amd import memory as mm

KINDS = (tsp.TSP_WS_MLP, tsp.TSP_WS_LAYER, tsp.TSP_WS_MLP_BWD, tsp.TSP_WS_ATTN_BWD, tsp.TSP_WS_LAYER_BWD)


def _lib_ws(m, kind):
    s = tsp.make_shape(m.S, m.D, m.r, m.h, m.H, m.Dh, m.F, dtype=m.dtype, rope_base=m.rope_base, Hkv=m.Hkv,
                       mlp=m.mlp)
    return tsp.workspace_size(s, kind)


SHAPES = [
    dict(S=1024, D=4, h=256, H=4, Dh=64, F=1024, dtype="f32"),       # the tiny fp32 layer
    dict(S=2048, D=4, h=512, H=4, Dh=128, F=1024),                    # small bf16 layer
    dict(S=384, D=2, h=256, H=4, Dh=64, F=512),                       # chunks of 96: 64 leading rows
    dict(S=64, D=2, h=256, H=4, Dh=64, F=256),                        # chunks of 16: fewer than 64 leading rows
    dict(S=131072, D=8, h=4096, H=32, Dh=128, F=16384),               # 7B
    dict(S=131072, D=8, h=4096, H=32, Dh=128, F=16384, Hkv=8, rope_base=5e5, mlp="swiglu"),
    dict(S=4096, D=1, h=1024, H=8, Dh=128, F=4096, mlp="swiglu"),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_workspace_matches_library(shape):
    for r in sorted({0, shape["D"] - 1}):
        m = mm.Model(r=r, **shape)
        for kind in KINDS:
            if kind == tsp.TSP_WS_MLP_BWD and (m.mlp != "gelu" or m.N % 64 != 0):
                continue  # the MLP backward covers the GELU MLP with S/D a multiple of 64
            if kind == tsp.TSP_WS_LAYER_BWD and (m.mlp != "gelu" or m.N % 64 != 0 or m.rope_base > 0):
                continue  # so does the layer backward, without rotation
            assert mm.workspace_bytes(m, kind) == _lib_ws(m, kind), (shape, r, kind)


def test_seven_b_components():
    m = mm.seven_b()
    rm = mm.rank_memory(m)
    # a layer's weights: QKV 3h^2, out-proj h^2, MLP 2hF, gains 2h (bf16)
    assert mm.layer_weight_elems(m) == 4 * 4096 ** 2 + 2 * 4096 * 16384 + 2 * 4096
    # the gathered K/V of one layer: S rows of K and V, all heads, bf16 --
    # the local eighth plus what the all-gather delivers
    full_kv = 131072 * 2 * 4096 * 2
    assert full_kv == 2 ** 31  # 2.15 GB
    assert rm["kv_gathered"] + rm["kv_local"] // m.layers == full_kv
    assert rm["kv_gathered"] == full_kv * 7 // 8
    # owned weights: 1/8 of the 32 layers
    assert rm["weights_owned"] == 32 * mm.layer_weight_elems(m) * 2 // 8
    assert rm["total"] == sum(v for k, v in rm.items() if k != "total")


def test_owned_memory_falls_as_one_over_d():
    """Paragraph 1: every rank holds 1/D of the weights and of the tokens, so
    parameter and activation memory fall by the same factor; the transients
    of one layer (the received shards, the gathered K/V rows) do not."""
    base = dict(S=131072, h=4096, H=32, Dh=128, F=16384, layers=32, r=1)
    one = mm.rank_memory(mm.Model(D=1, **base))
    for D in (2, 4, 8, 16):
        rmD = mm.rank_memory(mm.Model(D=D, **base))
        for key in ("weights_owned", "kv_local", "residual"):
            assert rmD[key] * D == one[key], (D, key)
        # the layer workspace holds [N][.] activations only (rank 1: no leading rows)
        assert rmD["workspace"] * D == one["workspace"], D
        assert rmD["weights_received"] == one["weights_owned"] // 32 * (D - 1) // D
        assert rmD["kv_gathered"] == 131072 * (D - 1) // D * 2 * 4096 * 2
    assert one["weights_received"] == 0 and one["kv_gathered"] == 0


def test_training_terms():
    m = mm.seven_b()
    fwd, trn = mm.rank_memory(m), mm.rank_memory(m, train=True)
    W = mm.layer_weight_elems(m)
    assert trn["grads_owned"] == 32 * W * 4 // 8
    assert trn["optimizer_owned"] == 3 * trn["grads_owned"]
    assert trn["saved_layer_inputs"] == 32 * m.N * m.h * 4
    for k in fwd:
        if k != "total":
            assert trn[k] == fwd[k]
    assert trn["total"] > fwd["total"]
    # one layer's backward: dK/dV over the sequence plus the rank's summed
    # rows, the library's layer-backward workspace, dy and dx, and the
    # received shards' weight gradients
    kvw = 2 * m.kv_heads * m.Dh
    assert trn["backward_peak"] == ((m.S + m.N) * kvw * 4 + _lib_ws(m, tsp.TSP_WS_LAYER_BWD) + 2 * m.N * m.h * 4
                                    + W * 4 * 7 // 8)
    # the training path that keeps each layer's attention output and
    # statistics and its MLP pre-activation (the buffers tsp_layer_fwd_save
    # fills): fp32 O and lse, Z
    sv = mm.rank_memory(m, train=True, save_attention=True)
    assert sv["saved_attention"] == 32 * (m.N * 4096 + 32 * m.N) * 4
    assert sv["saved_mlp_preact"] == 32 * m.N * 16384 * 2  # Z in bf16
    assert sv["total"] == trn["total"] + sv["saved_attention"] + sv["saved_mlp_preact"]


def test_single_gpu_bytes():
    """What a one-GPU run allocates: every shard and the whole gathered K/V
    resident, x and y, and the workspace."""
    for shape, layers in itertools.product(SHAPES[1:3], (1, 4)):
        m = mm.Model(layers=layers, **shape)
        e = 2 if m.dtype == "bf16" else 4
        want = (layers * (mm.layer_weight_elems(m) * e + m.S * 2 * m.kv_heads * m.Dh * e)
                + 2 * m.N * m.h * 4 + _lib_ws(m, tsp.TSP_WS_LAYER))
        assert mm.single_gpu_bytes(m, "layer") == want
        assert mm.single_gpu_bytes(m, "layers") == want + m.N * m.h * 4
