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


# Gradients of the bf16 layer backward. Every gradient passes through several
# operands rounded once to bf16 (unit roundoff u = 2^-8), and many are sums
# with cancellation whose elements differ in size by orders of magnitude
# from row to row (a key row seen by every query against one seen by a
# few), so an element's error scales with its own row, not with the
# tensor's rms. The rule is norm-wise: ||got - want|| <= TOL_BWD_BF16 *
# ||want|| over the tensor (2.5u; the rounding points give about u), and
# ||got_row - want_row|| <= TOL_BWD_BF16_ROW * ||want_row|| for every row
# along the first axis, the row norm floored at a tenth of the median row
# norm. A row that is a sum of few terms that cancel carries the terms'
# rounding error, not a fraction of its own size: a numpy emulation of the
# same rounding points reaches 6.4% on one key row of the 7B K gradient
# sampled over 14 queries. A wrong or missing row errs by about its whole
# size, and one missing term of seven by about 40%, so 25% still catches
# them. A row whose expected value is exactly zero (a query at position 0
# has dq = 0) is held to the floor alone: its rounding residue is not zero
# when Delta comes from the forward's stored output.
TOL_BWD_BF16 = 1e-2
TOL_BWD_BF16_ROW = 0.25


def assert_close_nw(got, want, what, tol=TOL_BWD_BF16, tol_row=TOL_BWD_BF16_ROW):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    if want.ndim > 1:
        G, W = got.reshape(want.shape[0], -1), want.reshape(want.shape[0], -1)
        wn = np.linalg.norm(W, axis=1)
        nz = wn[wn > 0]
        assert nz.size, f"{what}: expected tensor is zero"
        floor = 0.1 * float(np.median(nz))
        row = np.linalg.norm(G - W, axis=1) / np.maximum(wn, floor)
        worst = float(row.max())
        at = int(np.argmax(row))
        where = f" at row {at} (norm {wn[at]:.3e}, median {np.median(nz):.3e})"
    else:
        worst, where = err, ""
    log(f"  {what}: norm-wise err = {err:.3e} (tol {tol:g}), worst row = {worst:.3e}{where} (tol {tol_row:g})")
    assert err <= tol, f"{what}: norm-wise error {err:.3e} > {tol:g}"
    assert worst <= tol_row, f"{what}: a row's norm-wise error {worst:.3e} > {tol_row:g}"
    return err
