"""Pins of the oracle's backward (gradients of a loss through the causal forward).

The oracle's backward is the adjoint of its per-token recurrence.  It is pinned
to things other than itself:
- central finite differences of L = sum(dO * O) through the oracle's forward
  (itself pinned to the pages in test_oracle.py), for q, k, v and the initial
  state, gated and ungated, with both feature maps;
- the derivative of the masked quadratic form, derived separately by matrix
  calculus (oracle/quadratic.py);
- the one-token closed form: o = c v with c = s / (s + eps), s = phi(q).phi(k);
- linearity in dO.
"""
import numpy as np
import pytest

import oracle


def away_from_zero(x, margin=0.05):
    # keep inputs off the kink of phi at 0 so that central differences see one branch
    return np.where(np.abs(x) < margin, np.sign(x + 1e-300) * margin, x)


def inputs(B, H, N, Dk, Dv, gated=False, init=False, seed=0):
    r = np.random.default_rng(seed)
    q = away_from_zero(r.standard_normal((B, H, N, Dk)))
    k = away_from_zero(r.standard_normal((B, H, N, Dk)))
    v = r.standard_normal((B, H, N, Dv))
    do = r.standard_normal((B, H, N, Dv))
    a = r.uniform(0.3, 1.0, (B, H, N)) if gated else None
    s0 = r.standard_normal((B, H, Dk, Dv)) if init else None
    z0 = r.uniform(0.5, 2.0, (B, H, Dk)) if init else None
    return q, k, v, do, a, s0, z0


def loss(q, k, v, do, a, s0, z0, phi_mode):
    o, _, _ = oracle.forward(q, k, v, s0, z0, alpha=a, phi_mode=phi_mode)
    return float((o * do).sum())


def fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("phi_mode", [oracle.PHI_ELU1, oracle.PHI_IDENTITY])
def test_backward_matches_finite_differences(gated, phi_mode):
    q, k, v, do, a, s0, z0 = inputs(1, 2, 6, 3, 4, gated=gated, init=True, seed=7 + gated + 2 * phi_mode)
    if phi_mode == oracle.PHI_IDENTITY:
        # positive keys and queries keep the denominator away from zero
        q, k = np.abs(q), np.abs(k)
    dq, dk, dv, ds, dz = oracle.backward(q, k, v, do, s0, z0, alpha=a, phi_mode=phi_mode)
    f = lambda: loss(q, k, v, do, a, s0, z0, phi_mode)  # noqa: E731
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("s_init", s0, ds), ("z_init", z0, dz)):
        ref = fd_grad(f, x)
        scale = max(1.0, float(np.abs(ref).max()))
        assert np.abs(g - ref).max() <= 1e-6 * scale, (name, float(np.abs(g - ref).max()))


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("phi_mode", [oracle.PHI_ELU1, oracle.PHI_IDENTITY])
def test_backward_matches_the_quadratic_form(gated, phi_mode):
    q, k, v, do, a, _, _ = inputs(2, 2, 40, 8, 5, gated=gated, seed=11 + gated)
    if phi_mode == oracle.PHI_IDENTITY:
        q, k = np.abs(q), np.abs(k)
    got = oracle.backward(q, k, v, do, alpha=a, phi_mode=phi_mode)[:3]
    ref = oracle.quadratic_backward(q, k, v, do, a, phi_mode=phi_mode)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12, err_msg=name)


def test_one_token_closed_form():
    eps = 1e-3  # large enough that the eps terms are visible
    q, k, v, do, _, _, _ = inputs(1, 1, 1, 4, 3, seed=3)
    fq, fk = oracle.phi(q), oracle.phi(k)
    s = float((fq * fk).sum())
    c = s / (s + eps)
    dv_ref = c * do
    dc = float((do * v).sum())
    ds = dc * eps / (s + eps) ** 2
    dphi = lambda x: np.where(x >= 0, 1.0, np.exp(x))  # noqa: E731
    dq_ref = ds * fk * dphi(q)
    dk_ref = ds * fq * dphi(k)
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, eps=eps)
    np.testing.assert_allclose(dv, dv_ref, rtol=1e-12)
    np.testing.assert_allclose(dq, dq_ref, rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(dk, dk_ref, rtol=1e-10, atol=1e-15)


def test_linear_in_dout():
    q, k, v, do1, a, s0, z0 = inputs(1, 3, 30, 6, 7, gated=True, init=True, seed=5)
    do2 = np.random.default_rng(6).standard_normal(do1.shape)
    g1 = oracle.backward(q, k, v, do1, s0, z0, alpha=a)
    g2 = oracle.backward(q, k, v, do2, s0, z0, alpha=a)
    g12 = oracle.backward(q, k, v, do1 + 2.0 * do2, s0, z0, alpha=a)
    for x1, x2, x12 in zip(g1, g2, g12):
        np.testing.assert_allclose(x12, x1 + 2.0 * x2, rtol=1e-9, atol=1e-12)


def test_gate_of_one_equals_ungated_and_zero_gate_cuts_the_past():
    q, k, v, do, _, s0, z0 = inputs(1, 1, 12, 4, 4, init=True, seed=9)
    ones = np.ones((1, 1, 12))
    for x, y in zip(oracle.backward(q, k, v, do, s0, z0), oracle.backward(q, k, v, do, s0, z0, alpha=ones)):
        np.testing.assert_array_equal(x, y)
    # a zero gate at token 5 clears the summary: the later queries see nothing
    # of tokens 0..4 or of the initial state, so their gradients are those of
    # the first five tokens alone
    a = np.ones((1, 1, 12))
    a[0, 0, 5] = 0.0
    full = oracle.backward(q, k, v, do, s0, z0, alpha=a)
    head = oracle.backward(q[:, :, :5], k[:, :, :5], v[:, :, :5], do[:, :, :5], s0, z0, alpha=a[:, :, :5])
    for x, y in zip(full[:3], head[:3]):
        np.testing.assert_array_equal(x[:, :, :5], y)
    for x, y in zip(full[3:], head[3:]):
        np.testing.assert_array_equal(x, y)
