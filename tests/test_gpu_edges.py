"""GPU parity at the edges of the chunked kernels (eight-wave paths, Dk, Dv in {64, 128}).

Each case runs the library through the C ABI and compares element by element
with the fp64 oracle on the same seeded inputs:
- mixed head dims, causal and gated;
- one and two tokens, many heads with short sequences (no segment-state pass);
- lengths one row past or short of a chunk and of a segment boundary;
- the identity feature map on the bf16 chunk kernels (positive inputs, so the
  denominator stays away from zero), causal, gated and non-causal;
- ragged non-causal shapes.
"""
import pytest
import torch

import oracle
from linear_attention_phi_amd import binding as la
from linear_attention_phi_amd import synth
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF = torch.bfloat16


def make(B, H, N, Dk, Dv, seed, gated=False, positive=False, dtype=BF):
    w = synth.Workload("t", B, H, N, Dk, Dv, dtype, seed, q_scale=Dk ** -0.5, k_scale=Dk ** -0.5)
    q, k, v = synth.qkv(w)
    if positive:
        # |x| + 1/64, rounded once more to the input dtype: the identity map then
        # keeps every key and query positive, so phi(q).z > 0
        q, k = ((x.float().abs() + 1.0 / 64).to(dtype) for x in (q, k))
    a = synth.gate_heads(seed, B, H, N) if gated else None
    return q, k, v, a


def check(q, k, v, a=None, phi=la.PHI_ELU1):
    args = [x.to(DEV) for x in (q, k, v)]
    if a is None:
        o, s, z = la.linattn_forward(*args, phi=phi)
    else:
        o, s, z = la.linattn_forward_gated(*args, a.to(DEV), phi=phi)
    torch.cuda.synchronize()
    ro, rs, rz = oracle.forward(q, k, v, alpha=a, phi_mode=phi)
    tol = TOL[q.dtype]
    assert_close("O", o.cpu(), ro, tol)
    assert_close("S", s.cpu(), rs, tol, per="head")
    assert_close("z", z.cpu(), rz, tol, per="head")


@pytest.mark.parametrize("shape", [(2, 2, 900, 64, 128), (1, 2, 1300, 128, 64), (1, 1, 1, 128, 128),
                                   (1, 2, 2, 64, 64), (1, 1, 1, 64, 128), (16, 16, 100, 128, 128),
                                   (8, 4, 64, 128, 64)])
def test_forward_shapes(shape):
    q, k, v, _ = make(*shape, seed=800 + sum(shape))
    check(q, k, v)


@pytest.mark.parametrize("shape", [(1, 2, 900, 64, 128), (1, 1, 1300, 128, 64), (1, 1, 1, 128, 128),
                                   (16, 16, 100, 128, 128)])
def test_gated_shapes(shape):
    q, k, v, a = make(*shape, seed=820 + sum(shape), gated=True)
    check(q, k, v, a)


# Lengths around chunk (64) and segment multiples.  With one head the plan cuts
# the sequence into as many segments as there are chunks (up to 256), so these
# land one row before / after both kinds of boundary.
@pytest.mark.parametrize("N", [4095, 4097, 64 * 256 - 1, 64 * 256 + 1, 64 * 300 + 63])
def test_forward_boundaries(N):
    q, k, v, _ = make(1, 1, N, 128, 128, seed=840 + N % 97)
    check(q, k, v)


@pytest.mark.parametrize("N", [4097, 64 * 256 + 1])
def test_gated_boundaries(N):
    q, k, v, a = make(1, 1, N, 128, 128, seed=860 + N % 89, gated=True)
    check(q, k, v, a)


@pytest.mark.parametrize("shape", [(1, 2, 700, 128, 128), (1, 1, 333, 64, 128), (2, 1, 129, 128, 64)])
def test_identity_map_causal_and_gated(shape):
    q, k, v, a = make(*shape, seed=880 + sum(shape), gated=True, positive=True)
    check(q, k, v, None, phi=la.PHI_IDENTITY)
    check(q, k, v, a, phi=la.PHI_IDENTITY)


@pytest.mark.parametrize("shape,phi", [((1, 1, 65, 128, 128), la.PHI_ELU1), ((3, 2, 1, 64, 64), la.PHI_ELU1),
                                       ((1, 2, 4097, 128, 128), la.PHI_ELU1),
                                       ((1, 2, 700, 128, 128), la.PHI_IDENTITY)])
def test_noncausal_edges(shape, phi):
    q, k, v, _ = make(*shape, seed=900 + sum(shape), positive=phi == la.PHI_IDENTITY)
    o, s, z = la.linattn_forward_noncausal(q.to(DEV), k.to(DEV), v.to(DEV), phi=phi)
    torch.cuda.synchronize()
    ro, rs, rz = oracle.noncausal(q, k, v, phi_mode=phi)
    tol = TOL[q.dtype]
    assert_close("O", o.cpu(), ro, tol)
    assert_close("S", s.cpu(), rs, tol, per="head")
    assert_close("z", z.cpu(), rz, tol, per="head")
