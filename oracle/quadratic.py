"""Masked quadratic form of (gated) causal linear attention, NumPy fp64, tiny inputs only.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is the O(N^2) form that the state-space-models page compares against the
recurrence (section 2, "linear attention = recurrence", and its experiment B):

    o_t = sum_{j<=t} (phi(q_t) . phi(k_j)) v_j / sum_{j<=t} phi(q_t) . phi(k_j)

written as a score matrix masked to j <= t (diagonal included), times V,
divided row-wise by the masked row sums.  With a per-token decay a_t the score
of key j seen from query t is multiplied by prod_{m=j+1..t} a_m (the decay the
summary has received since token j was added).  ``causal=False`` drops the mask
and the decay.  eps is added to the denominator.
"""
from __future__ import annotations

import numpy as np


def _phi(x, mode):
    if mode == 1:
        return x
    return np.where(x >= 0, x, np.expm1(np.minimum(x, 0.0))) + 1.0


def quadratic_forward(q, k, v, alpha=None, *, eps=1e-6, phi_mode=0, causal=True):
    """q, k: [B, H, N, Dk]; v: [B, H, N, Dv]; alpha: [B, H, N] or None.  Returns O in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, _ = q.shape
    fq, fk = _phi(q, phi_mode), _phi(k, phi_mode)
    scores = np.matmul(fq, np.swapaxes(fk, -1, -2))  # [B, H, N(query), N(key)]
    if causal:
        weight = np.zeros((B, H, N, N))
        for b in range(B):
            for h in range(H):
                for t in range(N):
                    decay = 1.0
                    # walk back from the diagonal: key t is undecayed, key j has
                    # been multiplied by a_{j+1} ... a_t
                    for j in range(t, -1, -1):
                        weight[b, h, t, j] = scores[b, h, t, j] * decay
                        if alpha is not None:
                            decay *= float(alpha[b, h, j])
    else:
        weight = scores
    num = np.matmul(weight, v)
    den = weight.sum(axis=-1, keepdims=True)
    return num / (den + eps)
