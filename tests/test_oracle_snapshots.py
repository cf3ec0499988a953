"""Pins of the oracle's state snapshots (the summary after chosen tokens).

oracle.snapshots runs the pinned forward over each prefix.  It is checked
against things other than itself:
- ungated: S_p = phi(K_{0..p})^T V_{0..p} (one library matmul) and
  z_p = the column sums of phi(K_{0..p}), plus the initial state;
- gated: S_p = sum_j (a_{j+1} ... a_p) phi(k_j) v_j^T + (a_0 ... a_p) S_init,
  with the decay weights formed directly from the gates;
- resuming the forward from (S_p, z_p) on tokens p+1.. reproduces the full
  forward's outputs there, and the snapshot at N - 1 is the final state.
"""
import numpy as np
import pytest

import oracle


def inputs(B, H, N, Dk, Dv, seed, gated=False, init=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, N, Dk))
    k = r.standard_normal((B, H, N, Dk))
    v = r.standard_normal((B, H, N, Dv))
    a = r.uniform(0.2, 1.0, (B, H, N)) if gated else None
    s0 = r.standard_normal((B, H, Dk, Dv)) if init else None
    z0 = r.uniform(0.5, 2.0, (B, H, Dk)) if init else None
    return q, k, v, a, s0, z0


POS = [0, 1, 7, 15, 16, 30, 39]


@pytest.mark.parametrize("init", [False, True])
def test_ungated_snapshots_are_prefix_outer_products(init):
    q, k, v, _, s0, z0 = inputs(2, 2, 40, 5, 3, seed=21, init=init)
    s, z = oracle.snapshots(q, k, v, POS, s0, z0)
    fk = oracle.phi(k)
    for i, p in enumerate(POS):
        ref_s = np.matmul(np.swapaxes(fk[:, :, :p + 1], -1, -2), v[:, :, :p + 1])
        ref_z = fk[:, :, :p + 1].sum(axis=2)
        if init:
            ref_s, ref_z = ref_s + s0, ref_z + z0
        np.testing.assert_allclose(s[:, :, i], ref_s, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(z[:, :, i], ref_z, rtol=1e-12, atol=1e-12)


def test_gated_snapshots_are_decay_weighted_sums():
    q, k, v, a, s0, z0 = inputs(1, 2, 40, 4, 3, seed=22, gated=True, init=True)
    a[0, 1, 9] = 0.0  # an exact zero gate clears everything before token 9
    s, z = oracle.snapshots(q, k, v, POS, s0, z0, alpha=a)
    fk = oracle.phi(k)
    for i, p in enumerate(POS):
        for h in range(2):
            ref_s = np.prod(a[0, h, :p + 1]) * s0[0, h]
            ref_z = np.prod(a[0, h, :p + 1]) * z0[0, h]
            for j in range(p + 1):
                wgt = np.prod(a[0, h, j + 1:p + 1])
                ref_s = ref_s + wgt * np.outer(fk[0, h, j], v[0, h, j])
                ref_z = ref_z + wgt * fk[0, h, j]
            np.testing.assert_allclose(s[0, h, i], ref_s, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(z[0, h, i], ref_z, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("gated", [False, True])
def test_resume_from_a_snapshot_and_the_last_snapshot(gated):
    q, k, v, a, _, _ = inputs(1, 3, 50, 6, 4, seed=23, gated=gated)
    o, s_fin, z_fin = oracle.forward(q, k, v, alpha=a)
    pos = [19, 49]
    s, z = oracle.snapshots(q, k, v, pos, alpha=a)
    o2, _, _ = oracle.forward(q[:, :, 20:], k[:, :, 20:], v[:, :, 20:], s[:, :, 0], z[:, :, 0],
                              alpha=None if a is None else a[:, :, 20:])
    np.testing.assert_array_equal(o2, o[:, :, 20:])
    np.testing.assert_array_equal(s[:, :, 1], s_fin)
    np.testing.assert_array_equal(z[:, :, 1], z_fin)
