"""Pins of the fp64 oracle against what the pages and the mathematics fix.

CPU only.  Every function of ``oracle`` is checked against something other than
itself: values printed on the pages (``tests/golden``), closed forms, special
cases that reduce to a library routine, and brute force with the masked
quadratic form on tiny inputs.  ``test_oracle_mutants.py`` shows that planted
mistakes in the oracle's C source fail these pins.
"""
import math

import numpy as np
import pytest

import oracle
from conftest import golden

ID = oracle.PHI_IDENTITY
ELU = oracle.PHI_ELU1


def _bh(x):
    """Add the [B=1, H=1] leading axes."""
    return np.asarray(x, dtype=np.float64)[None, None]


# ---------------------------------------------------------------- feature map

def test_phi_closed_form():
    # elu(x) = x for x >= 0, exp(x) - 1 for x < 0; phi = elu + 1
    x = np.array([0.0, 1.0, -1.0, 2.5, -3.0, 1e-300, -1e-300, -700.0])
    y = oracle.phi(x)
    expect = [1.0, 2.0, math.exp(-1.0), 3.5, math.exp(-3.0), 1.0, 1.0, math.exp(-700.0)]
    np.testing.assert_allclose(y, expect, rtol=1e-15, atol=0)
    assert np.all(y > 0)
    # continuous at 0 from both sides
    eps = 1e-9
    left, right = oracle.phi(np.array([-eps, eps]))
    assert abs(left - 1.0) < 2e-9 and abs(right - 1.0) < 2e-9
    # identity mode is the identity
    z = np.linspace(-3, 3, 13)
    np.testing.assert_array_equal(oracle.phi(z, ID), z)


def test_phi_positive_on_random_inputs():
    x = np.random.default_rng(0).standard_normal(10000) * 5
    y = oracle.phi(x)
    assert np.all(y > 0)
    np.testing.assert_allclose(y[x >= 0], x[x >= 0] + 1, rtol=1e-15)
    np.testing.assert_allclose(y[x < 0], np.exp(x[x < 0]), rtol=1e-14)


# --------------------------------------------------- worked example: 2 x 2 state

def test_fixed_size_state_worked_example():
    g = golden("fixed_size_state_2x2.json")
    q, k, v = _bh(g["q"]), _bh(g["k"]), _bh(g["v"])
    printed = g["printed"]
    # state after each token: run the forward on the first t+1 tokens
    for t, expect in enumerate(printed["state_after_token"]):
        _, s, _ = oracle.forward(q[:, :, :t + 1], k[:, :, :t + 1], v[:, :, :t + 1],
                                 eps=0.0, phi_mode=ID)
        np.testing.assert_array_equal(s[0, 0], expect)
    o, s, z = oracle.forward(q, k, v, eps=0.0, phi_mode=ID)
    np.testing.assert_array_equal(z[0, 0], printed["z_final"])
    np.testing.assert_allclose(o[0, 0, 2], printed["y_last"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], g["derived"]["y"], rtol=0, atol=1e-15)
    # the read of the final state with the printed queries
    for qq, expect in printed["reads_of_final_state"]:
        np.testing.assert_array_equal(np.asarray(qq, float) @ s[0, 0], expect)
    # the denominator of the last output is the score sum (2), not the token count (3)
    assert np.asarray(g["q"][2], float) @ z[0, 0] == printed["denominator_last"]


def test_fixed_size_state_with_eps():
    g = golden("fixed_size_state_2x2.json")
    o, _, _ = oracle.forward(_bh(g["q"]), _bh(g["k"]), _bh(g["v"]), eps=1e-6, phi_mode=ID)
    np.testing.assert_allclose(o[0, 0, 2], [3 / (2 + 1e-6), 1 / (2 + 1e-6)], rtol=1e-15)


def test_outer_products():
    g = golden("fixed_size_state_2x2.json")
    for case in g["printed"]["outer_products"]:
        k = _bh([case["k"]])
        v = _bh([case["v"]])
        _, s, z = oracle.forward(k, k, v, eps=0.0, phi_mode=ID)
        np.testing.assert_allclose(s[0, 0], case["state"], rtol=1e-15, atol=0)
        np.testing.assert_allclose(z[0, 0], case["k"], rtol=1e-15)


def test_noncausal_worked_example():
    g = golden("fixed_size_state_2x2.json")
    o, s, z = oracle.noncausal(_bh(g["q"]), _bh(g["k"]), _bh(g["v"]), eps=0.0, phi_mode=ID)
    np.testing.assert_array_equal(s[0, 0], g["printed"]["noncausal_state"])
    np.testing.assert_allclose(o[0, 0], g["derived"]["noncausal_y"], rtol=0, atol=1e-15)
    # both product orders: (Q K^T) V equals Q (K^T V) before normalization
    Q, K, V = (np.asarray(g[x], float) for x in ("q", "k", "v"))
    np.testing.assert_array_equal((Q @ K.T) @ V, Q @ s[0, 0])


# ----------------------------------------- worked example: scalar values, no phi

def test_summary_scalar_example():
    g = golden("summary_scalar_values.json")
    keys = np.asarray(g["keys"], float)
    vals = np.asarray(g["values"], float)[:, None]
    p = g["printed"]
    _, s2, _ = oracle.forward(_bh(keys[:2]), _bh(keys[:2]), _bh(vals[:2]), eps=0.0, phi_mode=ID)
    np.testing.assert_allclose(s2[0, 0, :, 0], p["state_after_two"], rtol=0, atol=1e-15)
    for qq, r in p["reads_after_two"]:
        assert abs(np.asarray(qq, float) @ s2[0, 0, :, 0] - r) < 1e-12
    o, s3, z3 = oracle.forward(_bh(keys), _bh(keys), _bh(vals), eps=0.0, phi_mode=ID)
    np.testing.assert_allclose(s3[0, 0, :, 0], p["state_after_three"], rtol=1e-12)
    for qq, r in p["reads_after_three"]:
        assert abs(np.asarray(qq, float) @ s3[0, 0, :, 0] - r) < 1e-12
    np.testing.assert_allclose(z3[0, 0], g["derived"]["z_final"], rtol=1e-12)
    np.testing.assert_allclose(o[0, 0, :, 0], g["derived"]["o"], rtol=1e-12)


# ------------------------------------------------ brute force: quadratic form

@pytest.mark.parametrize("N,Dk,Dv,gated,seed", [
    (1, 4, 3, False, 1), (7, 5, 3, False, 2), (33, 16, 16, False, 3), (64, 16, 8, True, 4),
    (100, 8, 12, True, 5), (130, 32, 32, False, 6), (257, 16, 16, True, 7)])
def test_recurrence_equals_quadratic_form(N, Dk, Dv, gated, seed):
    rng = np.random.default_rng(seed)
    B, H = 2, 2
    q = rng.standard_normal((B, H, N, Dk))
    k = rng.standard_normal((B, H, N, Dk))
    v = rng.standard_normal((B, H, N, Dv))
    a = rng.uniform(0.3, 1.0, (B, H, N)) if gated else None
    o, _, _ = oracle.forward(q, k, v, alpha=a, eps=1e-6)
    oq = oracle.quadratic_forward(q, k, v, a, eps=1e-6)
    np.testing.assert_allclose(o, oq, rtol=1e-12, atol=1e-13)


def test_noncausal_equals_unmasked_quadratic_form():
    rng = np.random.default_rng(11)
    q, k = rng.standard_normal((2, 3, 2, 50, 12))
    v = rng.standard_normal((3, 2, 50, 9))
    o, _, _ = oracle.noncausal(q, k, v, eps=1e-6)
    np.testing.assert_allclose(o, oracle.quadratic_forward(q, k, v, eps=1e-6, causal=False),
                               rtol=1e-12, atol=1e-13)


# ------------------------------------------- final state: one library product

def test_final_state_is_one_contraction():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((2, 2, 3, 300, 24))
    v = rng.standard_normal((2, 3, 300, 20))
    _, s, z = oracle.forward(q, k, v, want_o=False)
    s2, z2 = oracle.state_from_prefix(k, v)
    np.testing.assert_allclose(s, s2, rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose(z, z2, rtol=1e-13)
    # and by an explicit sum of outer products on one head
    fk = np.where(k[1, 2] >= 0, k[1, 2] + 1, np.exp(k[1, 2]))
    np.testing.assert_allclose(s[1, 2], np.einsum("ti,tj->ij", fk, v[1, 2]), rtol=1e-12, atol=1e-10)
    _, sn, zn = oracle.noncausal(q, k, v)
    np.testing.assert_allclose(sn, s, rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose(zn, z, rtol=1e-13)


# ------------------------------------------------ split / resume and decode

def test_split_resume_is_exact():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((2, 1, 2, 90, 8))
    v = rng.standard_normal((1, 2, 90, 6))
    a = rng.uniform(0.5, 1, (1, 2, 90))
    for alpha in (None, a):
        o, s, z = oracle.forward(q, k, v, alpha=alpha)
        c = 37
        a1 = None if alpha is None else alpha[..., :c]
        a2 = None if alpha is None else alpha[..., c:]
        o1, s1, z1 = oracle.forward(q[..., :c, :], k[..., :c, :], v[..., :c, :], alpha=a1)
        o2, s2, z2 = oracle.forward(q[..., c:, :], k[..., c:, :], v[..., c:, :], s1, z1, alpha=a2)
        np.testing.assert_array_equal(np.concatenate([o1, o2], axis=2), o)
        np.testing.assert_array_equal(s2, s)
        np.testing.assert_array_equal(z2, z)


def test_decode_continues_forward():
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal((2, 2, 3, 41, 8))
    v = rng.standard_normal((2, 3, 41, 5))
    a = rng.uniform(0.5, 1, (2, 3, 41))
    for alpha in (None, a):
        o, s, z = oracle.forward(q, k, v, alpha=alpha)
        p1 = None if alpha is None else alpha[..., :40]
        _, sp, zp = oracle.forward(q[..., :40, :], k[..., :40, :], v[..., :40, :], alpha=p1)
        od, sd, zd = oracle.decode_step(q[..., 40, :], k[..., 40, :], v[..., 40, :], sp, zp,
                                        alpha=None if alpha is None else alpha[..., 40])
        np.testing.assert_array_equal(od, o[..., 40, :])
        np.testing.assert_array_equal(sd, s)
        np.testing.assert_array_equal(zd, z)


def test_decode_steps_reproduce_worked_states():
    g = golden("fixed_size_state_2x2.json")
    s = np.zeros((1, 1, 2, 2))
    z = np.zeros((1, 1, 2))
    for t in range(3):
        qq = np.asarray(g["q"][t], float)[None, None]
        kk = np.asarray(g["k"][t], float)[None, None]
        vv = np.asarray(g["v"][t], float)[None, None]
        o, s, z = oracle.decode_step(qq, kk, vv, s, z, eps=0.0, phi_mode=ID)
        np.testing.assert_array_equal(s[0, 0], g["printed"]["state_after_token"][t])
        np.testing.assert_allclose(o[0, 0], g["derived"]["y"][t], atol=1e-15)


# ------------------------------------------------------------ gated special cases

def test_gate_of_one_is_ungated():
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal((2, 2, 2, 60, 8))
    v = rng.standard_normal((2, 2, 60, 8))
    o, s, z = oracle.forward(q, k, v)
    og, sg, zg = oracle.forward(q, k, v, alpha=np.ones((2, 2, 60)))
    np.testing.assert_array_equal(og, o)
    np.testing.assert_array_equal(sg, s)
    np.testing.assert_array_equal(zg, z)


def test_gate_of_zero_keeps_only_the_current_token():
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal((2, 1, 1, 20, 6))
    v = rng.standard_normal((1, 1, 20, 4))
    o, _, _ = oracle.forward(q, k, v, alpha=np.zeros((1, 1, 20)), eps=1e-6)
    fq = np.where(q >= 0, q + 1, np.exp(q))
    fk = np.where(k >= 0, k + 1, np.exp(k))
    sc = (fq * fk).sum(-1, keepdims=True)
    np.testing.assert_allclose(o, v * sc / (sc + 1e-6), rtol=1e-13)


def test_decay_table_half_life_and_memory_length():
    t = golden("ssm_tables.json")["decay_table"]
    for a, half, mem in zip(t["a"], t["half_life_steps"], t["memory_length"]):
        # impulse: k_0 = v_0 = 1, later tokens zero, constant decay a
        n = 200
        k = np.zeros((1, 1, n, 1)); k[0, 0, 0, 0] = 1.0
        v = k.copy()
        q = np.ones((1, 1, n, 1))
        states = []
        for m in range(1, n + 1):
            _, s, _ = oracle.forward(q[:, :, :m], k[:, :, :m], v[:, :, :m],
                                     alpha=np.full((1, 1, m), a), phi_mode=ID)
            states.append(s[0, 0, 0, 0])
        states = np.array(states)  # states[t] = S after token t
        np.testing.assert_allclose(states, a ** np.arange(n), rtol=1e-12)
        assert int(np.argmax(states <= 0.5)) == half
        # constant input: z_N = sum_{t<N} a^t -> 1 / (1 - a)
        N = 6000
        ones = np.ones((1, 1, N, 1))
        _, _, z = oracle.forward(ones, ones, ones, alpha=np.full((1, 1, N), a), phi_mode=ID,
                                 want_o=False)
        np.testing.assert_allclose(z[0, 0, 0], mem, rtol=1e-9)


# ------------------------------------------------------------ argument checks

def test_oracle_rejects_bad_shapes():
    lib = oracle._load()
    rc = lib.oracle_forward(None, None, None, None, None, None, None, None, None,
                            1, 4, 2, 2, 0, 0.0, 1)
    assert rc == -1
