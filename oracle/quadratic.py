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


def _dphi(x, mode):
    # derivative of the feature map: 1 on x >= 0 and exp(x) on x < 0 for
    # elu + 1; 1 for the identity map
    if mode == 1:
        return np.ones_like(x)
    return np.where(x >= 0, 1.0, np.exp(np.minimum(x, 0.0)))


def _causal_mask(B, H, N, alpha):
    """M[t, j] = prod_{m=j+1..t} a_m for j <= t (1 without gates), 0 above the diagonal."""
    m = np.zeros((B, H, N, N))
    for b in range(B):
        for h in range(H):
            for t in range(N):
                decay = 1.0
                for j in range(t, -1, -1):
                    m[b, h, t, j] = decay
                    if alpha is not None:
                        decay *= float(alpha[b, h, j])
    return m


def quadratic_backward(q, k, v, dout, alpha=None, *, eps=1e-6, phi_mode=0):
    """Gradients (dq, dk, dv) of a loss through the masked quadratic form, given dout = dL/dO.

    Matrix calculus on O = (W V) / (W 1 + eps) with W = M * (phi(Q) phi(K)^T):
        dY = dout / den,  dd = -rowsum(dout * O) / den,
        dW = dY V^T + dd 1^T,
        dphi(Q) = (M * dW) phi(K),  dphi(K) = (M * dW)^T phi(Q),  dV = W^T dY,
    then the chain rule through phi.  No initial state; the gates are constants.
    """
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, H, N, _ = q.shape
    fq, fk = _phi(q, phi_mode), _phi(k, phi_mode)
    mask = _causal_mask(B, H, N, alpha)
    w = mask * np.matmul(fq, np.swapaxes(fk, -1, -2))
    den = w.sum(axis=-1, keepdims=True) + eps
    o = np.matmul(w, v) / den
    dy = dout / den
    dd = -(dout * o).sum(axis=-1, keepdims=True) / den
    dw = mask * (np.matmul(dy, np.swapaxes(v, -1, -2)) + dd)
    dfq = np.matmul(dw, fk)
    dfk = np.matmul(np.swapaxes(dw, -1, -2), fq)
    dv = np.matmul(np.swapaxes(w, -1, -2), dy)
    return dfq * _dphi(q, phi_mode), dfk * _dphi(k, phi_mode), dv
