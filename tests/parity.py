"""Shared helpers of the GPU parity tests: the error metric and tolerances.

Outputs cross zero, so a plain elementwise relative error is meaningless; the
metric is normwise per row: for every (b, h, t), max_j |got - ref| / max_j |ref|,
and the worst row is reported.  States are compared per head the same way,
snapshots per (b, h, position).  Where a row is by construction a small
difference of larger terms (a gradient whose two parts cancel), the row's
reference size is floored by the size of those terms, computed from the
oracle's quantities (``floor`` argument).
Tolerances: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""
import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def row_rel_err(got, ref, floor=None):
    """Worst over rows (last axis) of max|got - ref| / max(max|ref|, floor of the row)."""
    g, r = to64(got), to64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    num = np.abs(g - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    if floor is not None:
        den = np.maximum(den, to64(floor).reshape(den.shape))
    return float((num / np.maximum(den, 1e-30)).max())


def lead_rel_err(got, ref, lead):
    """Flatten everything after the first `lead` axes and compare each of those items."""
    g, r = to64(got), to64(ref)
    n = int(np.prod(g.shape[:lead]))
    return row_rel_err(g.reshape(n, -1), r.reshape(n, -1))


def head_rel_err(got, ref):
    """States: flatten everything after (B, H) and compare per head."""
    return lead_rel_err(got, ref, 2)


def assert_close(name, got, ref, tol, per="row", floor=None):
    """per: "row" (last axis), "head" (after B, H), "item" (after B, H and one more axis)."""
    if per == "row":
        err = row_rel_err(got, ref, floor)
    elif per == "head":
        err = head_rel_err(got, ref)
    elif per == "item":
        err = lead_rel_err(got, ref, 3)
    else:
        raise ValueError(per)
    print(f"  {name}: max {per}-relative error {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: error {err:.3e} > {tol:.0e}"
    return err


def dphi(x, phi):
    return np.ones_like(x) if phi == oracle.PHI_IDENTITY else np.where(x >= 0, 1.0, np.exp(x))


def dq_term_size(q, k, g, ro, s0=None, z0=None, phi=0, eps=1e-6):
    """max_j |dd_t z_t,j phi'(q_t,j)| per row, from the oracle's forward output ro."""
    q64, k64, g64 = (x.double().numpy() for x in (q, k, g))
    z = np.cumsum(oracle.phi(k64, phi), axis=2)
    if z0 is not None:
        z = z + z0.double().numpy()[:, :, None, :]
    den = (oracle.phi(q64, phi) * z).sum(-1) + eps
    dd = -(g64 * ro).sum(-1) / den
    return np.abs(dd[..., None] * z * dphi(q64, phi)).max(-1)
