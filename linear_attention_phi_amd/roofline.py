"""Algorithmic work and MI355X peaks: the denominators of every reported fraction.

Bytes count what the method itself must move (each input read once, each
output written once); flops count 2 per multiply-add.  Nothing here depends
on how a kernel is tiled.
"""
from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
HBM_BYTES_PER_S = 8.0e12
MFMA_BF16_FLOPS = 2.5e15
FP32_VECTOR_FLOPS = 157.3e12
CUS = 256
CLOCK_HZ = 2.4e9


def dtype_bytes(dtype) -> int:
    s = str(dtype)
    return 2 if ("bfloat16" in s or s in ("bf16", "1")) else 4


def forward_bytes(B, H, N, Dk, Dv, in_bytes, out_bytes=None, *, gated=False,
                  state_in=False, state_out=True) -> int:
    """Q, K, V read once, O written once, final (S, z) written once (fp32)."""
    out_bytes = in_bytes if out_bytes is None else out_bytes
    per_token = (2 * Dk + Dv) * in_bytes + Dv * out_bytes + (4 if gated else 0)
    state = (Dk * Dv + Dk) * 4
    return B * H * (N * per_token + state * (int(state_in) + int(state_out)))


def decode_bytes(B, H, Dk, Dv, in_bytes, out_bytes=None, *, gated=False, state_bytes=4) -> int:
    """(S, z) read and written once (fp32 unless state_bytes says otherwise), q/k/v read once, o written once."""
    out_bytes = in_bytes if out_bytes is None else out_bytes
    state = (Dk * Dv + Dk) * state_bytes
    return B * H * (2 * state + (2 * Dk + Dv) * in_bytes + Dv * out_bytes + (4 if gated else 0))


def backward_bytes(B, H, N, Dk, Dv, in_bytes) -> int:
    """Q, K, V, dO and the saved fp32 denominators read once; dQ, dK, dV written once."""
    return B * H * N * ((2 * Dk + 2 * Dv) * in_bytes + 4 + (2 * Dk + Dv) * in_bytes)


def backward_kernel_bytes(kernel, B, H, N, Dk, Dv, in_bytes) -> int | None:
    """What one launch of a whole-sequence backward kernel must move."""
    rows = B * H * N
    if kernel == "bwd_dq_bf16":  # q, k, v, dO, den in; dq, dd out
        return rows * ((3 * Dk + 2 * Dv) * in_bytes + 8)
    if kernel == "bwd_dkv_bf16":  # q, k, v, dO, den, dd in; dk, dv out
        return rows * ((3 * Dk + 3 * Dv) * in_bytes + 8)
    return None


def backward_kernel_flops(kernel, B, H, N, Dk, Dv) -> int | None:
    """Recurrence-level flops of a backward kernel (2 Dk Dv per token for each
    state-sized product): dQ pass S dY, the forward state update and the
    reverse sums of the state sub-segments (these skip the first segment of a
    sequence, so at P segments the figure is high by 2 Dk Dv N / P); dK/dV
    pass R v, R^T phi(k) and the reverse state update."""
    per = {"bwd_dq_bf16": 6, "bwd_dkv_bf16": 6}.get(kernel)
    return None if per is None else per * B * H * N * Dk * Dv


def backward_flops(B, H, N, Dk, Dv) -> int:
    """Per token, 2 Dk Dv each for: the forward state update (recomputed), S dY,
    the reverse state update, R v and R^T phi(k)."""
    return 10 * B * H * N * Dk * Dv


def delta_bytes(B, H, N, Dk, Dv, in_bytes) -> int:
    """Delta rule: Q, K, V read once, O written once, the final state written once (fp32)."""
    return B * H * (N * (2 * Dk + 2 * Dv) * in_bytes + Dk * Dv * 4)


def delta_flops(B, H, N, Dk, Dv) -> int:
    """Per token 2 Dk Dv each for the read with the key, the write and the read with the query."""
    return 6 * B * H * N * Dk * Dv


def method_flops(B, H, N, Dk, Dv) -> int:
    """Write S += phi(k) v^T and read phi(q)^T S per token: 2 Dk Dv each."""
    return 4 * B * H * N * Dk * Dv


def chunked_flops(B, H, N, Dk, Dv, C) -> int:
    """What a chunk-C kernel issues with full C x C score tiles (utilization check only)."""
    return B * H * N * (4 * Dk * Dv + 2 * C * Dk + 2 * C * Dv)


def quadratic_form_flops(N, D) -> int:
    """Score matrix then weighted sum, one contraction counted per form: 2 N^2 D."""
    return 2 * N * N * D


def recurrence_flops(N, D) -> int:
    """N state updates of D x D, one contraction counted: 2 N D^2."""
    return 2 * N * D * D


def hbm_time_s(nbytes) -> float:
    return nbytes / HBM_BYTES_PER_S
