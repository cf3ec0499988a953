"""Pins of the oracle's delta rule (read the summary with the key, write only the difference).

oracle.delta is checked against things other than itself:
- the product-order page's worked example (tests/golden/summary_scalar_values.json,
  section "The summary runs out of room"): from the summary (5, 3), the key
  (0.6, 0.8) reads 5.4, the difference to the value 10 is 4.6, the summary
  becomes (7.76, 6.68), re-reading with the key gives 10 and the query (1, 0)
  gives 7.76;
- beta = 0 writes nothing; orthogonal unit keys reduce it to the additive sum
  of outer products (one library matmul);
- with beta = 1 every write is an exact overwrite: reading right after with
  the same unit key returns the value; with beta in (0, 1) it returns
  (1 - beta) times the old read plus beta times the value;
- the key enters only through its direction (scaling it changes nothing);
- the feature map comes before the unit length: on inputs of one sign elu + 1
  is x + 1 or exp(x), so the elu + 1 run equals the identity-map run fed those
  values, and one token from a zero summary gives o = (kh . phi(q)) v with phi
  evaluated branch by branch.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "summary_scalar_values.json")))
ID = oracle.PHI_IDENTITY


def arr(x):
    return np.asarray(x, dtype=np.float64)


def test_worked_example():
    keys = arr(GOLD["keys"])            # [3, 2]
    vals = arr(GOLD["values"])[:, None]  # [3, 1]
    p = GOLD["printed"]["delta_rule"]
    q = np.stack([keys[0], keys[1], [1.0, 0.0]])  # the last read is the query (1, 0)
    o, s = oracle.delta(q[None, None], keys[None, None], vals[None, None], phi_mode=ID)
    np.testing.assert_allclose(s[0, 0, :, 0], p["state"], rtol=1e-14)
    np.testing.assert_allclose(o[0, 0, 2, 0], p["read_with_1_0"], rtol=1e-14)
    # the two orthogonal keys first reproduce the additive state (5, 3)
    _, s2 = oracle.delta(q[None, None, :2], keys[None, None, :2], vals[None, None, :2], phi_mode=ID)
    np.testing.assert_allclose(s2[0, 0, :, 0], GOLD["printed"]["state_after_two"], rtol=1e-14)
    # from (5, 3): a zero-beta token reads with the key (5.4); a full write
    # adds difference (4.6) times the key, and re-reading gives the value
    k3 = keys[2][None, None, None]
    s0 = s2
    o_read, s_same = oracle.delta(k3, k3, arr([[[[10.0]]]]), beta=arr([[[0.0]]]), s_init=s0, phi_mode=ID)
    np.testing.assert_allclose(o_read[0, 0, 0, 0], p["read_before_write"], rtol=1e-14)
    np.testing.assert_array_equal(s_same, s0)
    o_re, s3 = oracle.delta(k3, k3, arr([[[[10.0]]]]), s_init=s0, phi_mode=ID)
    np.testing.assert_allclose((s3 - s0)[0, 0, :, 0], p["difference"] * keys[2], rtol=1e-13)
    np.testing.assert_allclose(o_re[0, 0, 0, 0], p["reread"], rtol=1e-14)


def rand(B, H, N, Dk, Dv, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((B, H, N, Dk)), r.standard_normal((B, H, N, Dk)), r.standard_normal((B, H, N, Dv))


def test_zero_beta_writes_nothing():
    q, k, v = rand(1, 2, 20, 5, 3, seed=31)
    s0 = np.random.default_rng(32).standard_normal((1, 2, 5, 3))
    o, s = oracle.delta(q, k, v, beta=np.zeros((1, 2, 20)), s_init=s0)
    np.testing.assert_array_equal(s, s0)
    np.testing.assert_allclose(o, np.matmul(oracle.phi(q), s0), rtol=1e-12)


def test_orthogonal_unit_keys_reduce_to_the_additive_sum():
    D, Dv = 6, 4
    r = np.random.default_rng(33)
    basis = np.linalg.qr(r.standard_normal((D, D)))[0]  # orthonormal rows
    k = basis[r.permutation(D)][None, None]              # each direction once
    v = r.standard_normal((1, 1, D, Dv))
    q = r.standard_normal((1, 1, D, D))
    o, s = oracle.delta(q, k, v, phi_mode=ID)
    ref_s = np.matmul(np.swapaxes(k, -1, -2), v)
    np.testing.assert_allclose(s, ref_s, rtol=1e-12, atol=1e-12)
    ref_o = np.stack([q[0, 0, t] @ np.matmul(k[0, 0, :t + 1].T, v[0, 0, :t + 1]) for t in range(D)])
    np.testing.assert_allclose(o[0, 0], ref_o, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("beta_const", [1.0, 0.3])
def test_each_write_overwrites_along_its_key(beta_const):
    # identity map; query t = the unit key t, so o_t is the read right after the write
    q, k, v = rand(1, 1, 30, 8, 5, seed=34)
    kh = k / np.linalg.norm(k, axis=-1, keepdims=True)
    beta = np.full((1, 1, 30), beta_const)
    o, _ = oracle.delta(kh, k, v, beta=beta, phi_mode=ID)
    # the read before the write, from the states of the prefix runs
    for t in range(30):
        _, s_prev = oracle.delta(kh[:, :, :t], k[:, :, :t], v[:, :, :t], beta=beta[:, :, :t], phi_mode=ID)
        read_before = kh[0, 0, t] @ s_prev[0, 0]
        ref = (1 - beta_const) * read_before + beta_const * v[0, 0, t]
        np.testing.assert_allclose(o[0, 0, t], ref, rtol=1e-10, atol=1e-10)


def test_only_the_key_direction_matters():
    q, k, v = rand(2, 1, 25, 4, 3, seed=35)
    scale = np.random.default_rng(36).uniform(0.1, 10.0, (2, 1, 25, 1))
    for mode in (ID,):
        o1, s1 = oracle.delta(q, k, v, phi_mode=mode)
        o2, s2 = oracle.delta(q, k * scale, v, phi_mode=mode)
        np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(s2, s1, rtol=1e-10, atol=1e-12)


# ---- the gated form (the same section: Gated DeltaNet, a global decay combined with the overwrite)

def test_gate_of_one_is_the_plain_rule():
    q, k, v = rand(1, 2, 30, 6, 4, seed=37)
    o1, s1 = oracle.delta(q, k, v)
    o2, s2 = oracle.delta(q, k, v, alpha=np.ones((1, 2, 30)))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_zero_gate_forgets_everything_before():
    # a_t = 0 clears the summary: from token t on, the run equals a fresh run
    # started at t (u_t = 0, S_t = beta_t kh_t v_t^T)
    q, k, v = rand(1, 1, 40, 5, 3, seed=38)
    a = np.random.default_rng(39).uniform(0.5, 1.0, (1, 1, 40))
    a[0, 0, 17] = 0.0
    s0 = np.random.default_rng(40).standard_normal((1, 1, 5, 3))
    o, s = oracle.delta(q, k, v, alpha=a, s_init=s0)
    o_tail, s_tail = oracle.delta(q[:, :, 17:], k[:, :, 17:], v[:, :, 17:], alpha=np.concatenate(
        [np.ones((1, 1, 1)), a[:, :, 18:]], axis=2))
    np.testing.assert_allclose(o[:, :, 17:], o_tail, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, s_tail, rtol=1e-12, atol=1e-12)


def test_gated_orthogonal_unit_keys_are_the_decayed_sum():
    # distinct orthonormal keys never read each other, so the state is the
    # additive sum of outer products, each decayed by the gates after it
    D, Dv = 6, 3
    r = np.random.default_rng(41)
    basis = np.linalg.qr(r.standard_normal((D, D)))[0]
    k = basis[r.permutation(D)][None, None]
    v = r.standard_normal((1, 1, D, Dv))
    a = r.uniform(0.3, 1.0, (1, 1, D))
    _, s = oracle.delta(k, k, v, alpha=a, phi_mode=ID)
    ref = sum(np.prod(a[0, 0, j + 1:]) * np.outer(k[0, 0, j], v[0, 0, j]) for j in range(D))
    np.testing.assert_allclose(s[0, 0], ref, rtol=1e-12, atol=1e-12)


# ---- the feature map inside the delta rule: phi first, then the unit length
# (product-order page, "The summary runs out of room": the key the summary is
# read and written with is the feature-mapped key; it has unit length, which is
# what makes the re-read return the value).  elu + 1 is x + 1 on x >= 0 and
# exp(x) on x < 0, so on inputs of one sign the elu + 1 run must equal the
# identity-map run fed those values directly; applying phi after the
# normalization (or to the query differently) breaks it.

def test_elu_mode_on_nonnegative_inputs_is_the_identity_run_on_x_plus_one():
    r = np.random.default_rng(42)
    q, k, v = (np.abs(x) for x in rand(2, 2, 30, 6, 4, seed=43))
    v = v * r.choice([-1.0, 1.0], v.shape)  # values keep both signs (phi never touches them)
    beta = r.uniform(0.2, 1.0, (2, 2, 30))
    a = r.uniform(0.6, 1.0, (2, 2, 30))
    s0 = r.standard_normal((2, 2, 6, 4))
    o1, s1 = oracle.delta(q, k, v, beta=beta, s_init=s0, alpha=a)
    o2, s2 = oracle.delta(q + 1.0, k + 1.0, v, beta=beta, s_init=s0, alpha=a, phi_mode=ID)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)


def test_elu_mode_on_negative_inputs_is_the_identity_run_on_exp():
    r = np.random.default_rng(44)
    q, k, v = rand(1, 3, 25, 5, 3, seed=45)
    q, k = -np.abs(q) - 1e-3, -np.abs(k) - 1e-3
    beta = r.uniform(0.2, 1.0, (1, 3, 25))
    o1, s1 = oracle.delta(q, k, v, beta=beta)
    o2, s2 = oracle.delta(np.exp(q), np.exp(k), v, beta=beta, phi_mode=ID)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)


def test_elu_mode_one_token_closed_form():
    # from a zero summary one full write leaves kh v^T, so o = (kh . phi(q)) v with
    # kh = phi(k) / |phi(k)|; phi here is evaluated branch by branch by hand
    k = arr([[[[0.5, -1.0, 2.0, -0.25]]]])
    q = arr([[[[-0.5, 0.0, 1.5, -2.0]]]])
    v = arr([[[[3.0, -1.0]]]])
    fk = np.array([1.5, np.exp(-1.0), 3.0, np.exp(-0.25)])
    fq = np.array([np.exp(-0.5), 1.0, 2.5, np.exp(-2.0)])
    kh = fk / np.sqrt((fk ** 2).sum())
    o, s = oracle.delta(q, k, v)
    np.testing.assert_allclose(s[0, 0], np.outer(kh, v[0, 0, 0]), rtol=1e-14)
    np.testing.assert_allclose(o[0, 0, 0], (kh @ fq) * v[0, 0, 0], rtol=1e-14)
