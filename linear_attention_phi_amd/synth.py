"""Seeded synthetic inputs, shared by the tests, the benchmark and the oracle checks.

This module draws random numbers, scales them and rounds them to the storage
dtype.  It holds none of the method's arithmetic (no feature map, no state, no
read), so the HIP path and the oracle can both consume its output without
sharing any code of the method.

Recipe (the same for every workload):

* Each (tensor, batch, head) has its own stream: NumPy ``PCG64`` seeded by
  ``SeedSequence(entropy=seed, spawn_key=(tensor_id, b, h))``.  Any single head
  can therefore be regenerated alone, and streams are filled in parallel.
* A stream draws ``standard_normal`` in float32, row-major over [N, D]
  (token-major), multiplies by the workload's scale in float32 and rounds to
  the storage dtype (bf16 with round-to-nearest-even, or fp32 as is).
* Decay gates draw ``g ~ N(4, 1)`` in float64 and store ``alpha = sigmoid(g)``
  rounded once to float32.

Tensor ids: 0 = Q, 1 = K, 2 = V, 3 = gate g, 4 = prefix K, 5 = prefix V.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

Q_ID, K_ID, V_ID, G_ID, PK_ID, PV_ID, DO_ID = 0, 1, 2, 3, 4, 5, 6


def _stream(seed: int, tensor_id: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=seed, spawn_key=(tensor_id, b, h))))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_heads(seed: int, tensor_id: int, B: int, H: int, N: int, D: int,
                 scale: float = 1.0, dtype: torch.dtype = torch.bfloat16,
                 heads=None) -> torch.Tensor:
    """[B, H, N, D] (or [len(heads), N, D] for an explicit list of (b, h)) of N(0,1)*scale."""
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    out32 = np.empty((len(pairs), N, D), dtype=np.float32)
    sc = np.float32(scale)

    def fill(i):
        b, h = pairs[i]
        _stream(seed, tensor_id, b, h).standard_normal(out=out32[i].reshape(-1), dtype=np.float32)
        if scale != 1.0:
            np.multiply(out32[i], sc, out=out32[i])

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(len(pairs))))
    t = torch.from_numpy(out32)
    if dtype != torch.float32:
        t = t.to(dtype)
    if heads is None:
        t = t.reshape(B, H, N, D)
    return t


def gate_heads(seed: int, B: int, H: int, N: int, mean: float = 4.0, heads=None) -> torch.Tensor:
    """alpha = sigmoid(g), g ~ N(mean, 1), as float32 [B, H, N] (or [len(heads), N])."""
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    out = np.empty((len(pairs), N), dtype=np.float32)

    def fill(i):
        b, h = pairs[i]
        g = _stream(seed, G_ID, b, h).standard_normal(N) + mean
        out[i] = (1.0 / (1.0 + np.exp(-g))).astype(np.float32)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(len(pairs))))
    t = torch.from_numpy(out)
    return t.reshape(B, H, N) if heads is None else t


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype, scales and seed."""
    name: str
    B: int
    H: int
    N: int
    Dk: int
    Dv: int
    dtype: torch.dtype
    seed: int
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    gated: bool = False
    decode: bool = False
    prefix: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.B * (1 if self.decode else self.N)


_R128 = 1.0 / math.sqrt(128.0)

# The five workloads the method is measured and checked on.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 64, 16, 16, torch.float32, 1001),
    "b4h8_n4096_d64": Workload("b4h8_n4096_d64", 4, 8, 4096, 64, 64, torch.bfloat16, 1002,
                               q_scale=1.0 / 8.0, k_scale=1.0 / 8.0),
    "long_n131072_d128": Workload("long_n131072_d128", 1, 16, 131072, 128, 128, torch.bfloat16,
                                  1003, q_scale=_R128, k_scale=_R128, v_scale=_R128),
    "decode_b256h32_d128": Workload("decode_b256h32_d128", 256, 32, 1, 128, 128, torch.bfloat16,
                                    1004, q_scale=_R128, k_scale=_R128, v_scale=_R128,
                                    decode=True, prefix=2048),
    "gated_b2h16_n16384_d128": Workload("gated_b2h16_n16384_d128", 2, 16, 16384, 128, 128,
                                        torch.bfloat16, 1005, q_scale=_R128, k_scale=_R128,
                                        v_scale=_R128, gated=True),
    # delta rule: unscaled q, k (elu + 1 of N(0, 1), so that the unit keys are
    # far from all parallel), 256 heads (one workgroup each)
    "delta_b16h16_n4096_d128": Workload("delta_b16h16_n4096_d128", 16, 16, 4096, 128, 128,
                                        torch.bfloat16, 1006),
}


def qkv(w: Workload, heads=None, N=None):
    """Q, K, V of a workload (all heads, or the listed (b, h) pairs); N overrides the length."""
    n = w.N if N is None else N
    q = normal_heads(w.seed, Q_ID, w.B, w.H, n, w.Dk, w.q_scale, w.dtype, heads)
    k = normal_heads(w.seed, K_ID, w.B, w.H, n, w.Dk, w.k_scale, w.dtype, heads)
    v = normal_heads(w.seed, V_ID, w.B, w.H, n, w.Dv, w.v_scale, w.dtype, heads)
    return q, k, v


def dout(w: Workload, heads=None, N=None) -> torch.Tensor:
    """An upstream gradient dL/dO for the backward: N(0, 1) in the workload's dtype, [B, H, N, Dv]."""
    n = w.N if N is None else N
    return normal_heads(w.seed, DO_ID, w.B, w.H, n, w.Dv, 1.0, w.dtype, heads)


def alpha(w: Workload, heads=None, N=None) -> torch.Tensor:
    return gate_heads(w.seed, w.B, w.H, w.N if N is None else N, heads=heads)


def decode_token(w: Workload):
    """The new token of a decode workload: q, k [B, H, Dk], v [B, H, Dv]."""
    q, k, v = qkv(w, N=1)
    return q[:, :, 0], k[:, :, 0], v[:, :, 0]


def decode_prefix(w: Workload, b: int):
    """Prefix keys and values of batch row b: [H, prefix, Dk], [H, prefix, Dv]."""
    heads = [(b, h) for h in range(w.H)]
    k = normal_heads(w.seed, PK_ID, w.B, w.H, w.prefix, w.Dk, w.k_scale, w.dtype, heads)
    v = normal_heads(w.seed, PV_ID, w.B, w.H, w.prefix, w.Dv, w.v_scale, w.dtype, heads)
    return k, v
