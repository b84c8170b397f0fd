"""tsp_zigzag_attn_bwd_noalloc, the attention backward that allocates
nothing (its row statistics live in the library's static device array),
against tsp_zigzag_attn_bwd with a caller workspace: identical outputs, bit
for bit (the same kernels on the same inputs), on two calls in a row, the
second with a smaller input, so that the second call runs over the first
call's leftovers in the array. Also: a shape beyond the array is rejected
with nothing enqueued."""
import numpy as np
import pytest

import synth
import tsp_rank_local_amd as tsp
from gpu_util import log, torch_cuda, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_cuda()
    tsp.lib()
    return t


def _run(torch, S, D, r, H, Hkv, Dh, dtype, seed):
    shape = synth.LayerShape(S=S, D=D, h=H * Dh, H=H, Dh=Dh, F=64 * D, dtype=dtype, Hkv=Hkv)
    N = S // D
    k, v = synth.remote_kv(shape, seed=seed)
    q = synth.normal((N, H, Dh), seed, synth.TID_Q, r, dtype=dtype)
    do = synth.normal((N, H, Dh), seed, synth.TID_DY, r, dtype=dtype)
    s = tsp.make_shape(S, D, r, H * Dh, H, Dh, 64 * D, dtype=dtype, Hkv=Hkv)
    qd, kd, vd, dod = up(q, dtype), up(k, dtype), up(v, dtype), up(do, dtype)
    kvh = Hkv or H

    def outs():
        return (torch.full((N, H, Dh), float("nan"), dtype=torch.float32, device="cuda"),
                torch.full((S, kvh, Dh), float("nan"), dtype=torch.float32, device="cuda"),
                torch.full((S, kvh, Dh), float("nan"), dtype=torch.float32, device="cuda"))

    ref, got = outs(), outs()
    ws = torch.empty(tsp.workspace_size(s, tsp.TSP_WS_ATTN_BWD), dtype=torch.uint8, device="cuda")
    log(f"attention backward with and without a workspace: S={S} D={D} r={r} H={H} Hkv={Hkv} Dh={Dh} {dtype}")
    tsp.tsp_zigzag_attn_bwd(s, qd, kd, vd, dod, *ref, ws)
    tsp.tsp_zigzag_attn_bwd_noalloc(s, qd, kd, vd, dod, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert bool(torch.isfinite(a).all()), name
        assert torch.equal(a, b), f"{name}: outputs differ"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_call_twice(torch, dtype):
    if dtype == "bf16":
        _run(torch, 4096, 4, 1, 8, 2, 128, dtype, seed=61)   # first call: H*N = 8192 statistics
        _run(torch, 1024, 2, 1, 4, 4, 64, dtype, seed=62)    # second, smaller: 2048, over the first's leftovers
    else:
        _run(torch, 1024, 4, 2, 4, 4, 64, dtype, seed=63)
        _run(torch, 256, 2, 0, 2, 1, 64, dtype, seed=64)


def test_noalloc_7b_shape_fits_and_larger_is_rejected(torch):
    # the 7B shape (H * S/D = 524288) fits in the 8 MiB array; four times that does not
    s7 = tsp.make_shape(131072, 8, 0, 4096, 32, 128, 16384, dtype="bf16")
    assert tsp.workspace_size(s7, tsp.TSP_WS_ATTN_BWD) <= 8 << 20
    big = tsp.make_shape(524288, 8, 0, 4096, 32, 128, 16384, dtype="bf16")
    x = torch.empty(16, dtype=torch.float32, device="cuda")
    p = x.data_ptr()
    with pytest.raises(tsp.TspError) as ei:
        tsp.tsp_zigzag_attn_bwd_noalloc(big, p, p + (1 << 40), p + (2 << 40), p + (3 << 40), p + (4 << 40),
                                        p + (5 << 40), p + (6 << 40))
    assert ei.value.status == tsp.TSP_ERR_UNSUPPORTED
    assert b"static" in tsp.lib().tsp_last_error()
    torch.cuda.synchronize()
