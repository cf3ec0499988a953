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


def row_errors(got, ref, floor=None):
    """Per row (last axis): (max|got - ref|, max|ref|, the row's reference size used)."""
    g, r = to64(got), to64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    num = np.abs(g - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    size = den if floor is None else np.maximum(den, to64(floor).reshape(den.shape))
    return num, den, size


def row_rel_err(got, ref, floor=None):
    """Worst over rows (last axis) of max|got - ref| / max(max|ref|, floor of the row)."""
    g = to64(got)
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    num, _, size = row_errors(got, ref, floor)
    return float((num / np.maximum(size, 1e-30)).max())


def worst_rows(got, ref, floor=None, n=6):
    """Lines describing the n worst rows (index, error, row size, floor), for failure reports."""
    num, den, size = row_errors(got, ref, floor)
    rel = num / np.maximum(size, 1e-30)
    idx = np.argsort(rel.reshape(-1))[::-1][:n]
    out = []
    for i in idx:
        at = np.unravel_index(i, rel.shape)
        fl = "" if floor is None else f" floor {to64(floor).reshape(rel.shape)[at]:.3e}"
        out.append(f"    row {tuple(int(x) for x in at)}: err {num[at]:.3e} |ref| {den[at]:.3e}{fl} rel {rel[at]:.3e}")
    return out


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
    if err > tol and per == "row" and np.isfinite(err):
        print("\n".join(worst_rows(got, ref, floor)), flush=True)
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


def dk_term_size(q, k, v, g, ro, s0=None, z0=None, phi=0, eps=1e-6):
    """Root-sum-square of the elementary products each dk row sums, max over the row.

    dk_t,i = phi'(k_t,i) sum_{u >= t} phi(q_u,i) sum_j dY_u,j (v_t,j - o_u,j)
    (dY_u = dO_u / den_u; the o_u part is dd_u = -(dO_u . o_u) / den_u).  The
    row's columns share every scalar factor (phi(q) is near one), so a whole
    row can be a sum of products of either sign that ends near zero -- over
    the later tokens u, and within each dot product over j (the last token's
    row is one such dot product).  Its rounding error scales with the size of
    those products, sqrt(sum_u phi(q_u)^2 sum_j dY_u,j^2 (v_t,j^2 + o_u,j^2)),
    not with the row; phi(q_u)^2 is bounded by its maximum over the columns.
    """
    q64, k64, v64, g64 = (x.double().numpy() for x in (q, k, v, g))
    z = np.cumsum(oracle.phi(k64, phi), axis=2)
    if z0 is not None:
        z = z + z0.double().numpy()[:, :, None, :]
    fq = oracle.phi(q64, phi)
    den = (fq * z).sum(-1) + eps
    dy2 = (g64 / den[..., None]) ** 2
    w = (fq ** 2).max(-1, keepdims=True)
    # suffix sums over u >= t
    a = np.flip(np.cumsum(np.flip(w * dy2, 2), 2), 2)                      # [B, H, N, Dv]
    b = np.flip(np.cumsum(np.flip((w * dy2 * ro ** 2).sum(-1), 2), 2), 2)  # [B, H, N]
    return np.sqrt((v64 ** 2 * a).sum(-1) + b) * np.abs(dphi(k64, phi)).max(-1)
