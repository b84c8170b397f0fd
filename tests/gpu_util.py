"""Helpers for the GPU parity tests: device upload/download and the tolerance
rule (max |err| <= tol * rms(expected), rms over the compared oracle values)."""
import sys

import numpy as np

import synth

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("needs a GPU")
    return torch


def up(a, dtype):
    """numpy (float32, or uint16 bf16 bits) -> device tensor."""
    import tsp_rank_local_amd as tsp
    return tsp.to_device(a, dtype)


def down(t):
    """device tensor -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(a, dtype):
    """Stored host tensor -> float64 values (bf16 widened exactly)."""
    return synth.as_f32(a, dtype).astype(np.float64)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_close(got, want, tol, what, rms=None):
    """max |got - want| <= tol * rms(want); rms may be given (stratified estimate)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if rms is None:
        rms = float(np.sqrt(np.mean(want * want)))
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    log(f"  {what}: max|err| = {err:.3e}, rms = {rms:.3e}, ratio = {err / max(rms, 1e-300):.3e} (tol {tol:g})")
    assert err <= tol * rms, f"{what}: max|err| {err:.3e} > {tol:g} * rms {rms:.3e}"
    return err / rms
