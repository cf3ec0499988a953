"""Shared helpers of the GPU parity tests: the error metric and tolerances.

Outputs cross zero, so a plain elementwise relative error is meaningless; the
metric is normwise per row: for every (b, h, t), max_j |got - ref| / max_j |ref|,
and the worst row is reported.  States are compared per head the same way.
Tolerances: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def row_rel_err(got, ref, floor=1e-30):
    """Worst over rows (last axis) of max|got - ref| / max|ref|."""
    g, r = to64(got), to64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    num = np.abs(g - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float((num / np.maximum(den, floor)).max())


def head_rel_err(got, ref):
    """States: flatten everything after (B, H) and compare per head."""
    g, r = to64(got), to64(ref)
    return row_rel_err(g.reshape(g.shape[0] * g.shape[1], -1), r.reshape(r.shape[0] * r.shape[1], -1))


def assert_close(name, got, ref, tol, per="row"):
    err = row_rel_err(got, ref) if per == "row" else head_rel_err(got, ref)
    print(f"  {name}: max {per}-relative error {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: error {err:.3e} > {tol:.0e}"
    return err
