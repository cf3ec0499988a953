"""GPU parity of the backward (dq, dk, dv) against the fp64 oracle's adjoint.

The training forward runs through the C ABI (its o must agree with the plain
forward's), the backward takes its den (and, unless a test says otherwise, its
saved segment states), and every gradient is
compared with oracle.backward on the same seeded inputs (the oracle uses the
exact forward, so the comparison includes every rounding of the kernels).

Every gradient row (b, h, t) is compared normwise, max_j |got - ref| /
max_j |ref|, at the bf16 tolerance; the head-normwise figure is printed as well.
dq is a difference of two terms that cancel along phi(q): phi(q_t) . dphi(q_t)
= 0 up to eps, and at a sequence's first token o = v whatever q is, so the
exact dq there is eps-sized.  Each dq row's reference size is therefore floored
by the size of one of the two terms it is the difference of, |dd_t z_t phi'(q_t)|
(dd_t = -(dO_t . o_t) / den_t, z_t the running key sum), formed from the
oracle's forward.  A dk row is a double sum,
phi'(k_t) sum_{u >= t} phi(q_u) sum_j dY_u,j (v_t,j - o_u,j), whose columns
share every scalar factor (phi(q) is near one): the whole row can be a sum of
products of either sign that ends near zero (at the last token it is a single
dot product over the value columns), and its rounding error scales with the
products, not with the row.  Each dk row is therefore floored by the
root-sum-square of those products (parity.dk_term_size; a dropped or doubled
chunk of 64 tokens is still about 15x above that floor at 2e-2).  dv rows have
independent columns and are compared plainly.  Every gradient must also meet
the tolerance head-normwise.  Shapes span several chunks and segments (the reverse segment
sums), ragged tails, both head dims and their mix, and inputs with and without the 1/sqrt(D)
scale (features and denominators over a wider range).  Sequences of one token get
their own test: there every row of dq and dk is eps-sized.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_phi_amd import binding as la
from linear_attention_phi_amd import synth
from parity import TOL, assert_close, dk_term_size, dq_term_size

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def make(B, H, N, Dk, Dv, seed, positive=False, scale=None):
    s = Dk ** -0.5 if scale is None else scale
    w = synth.Workload("t", B, H, N, Dk, Dv, torch.bfloat16, seed, q_scale=s, k_scale=s)
    q, k, v = synth.qkv(w)
    if positive:
        q, k = ((x.float().abs() + 1.0 / 64).to(torch.bfloat16) for x in (q, k))
    return q, k, v, synth.dout(w)


def run(q, k, v, g, phi=la.PHI_ELU1, s0=None, z0=None, use_saved=True):
    """use_saved: the backward reads the training forward's segment states (else recomputes them)."""
    d = [x.to(DEV) for x in (q, k, v, g)]
    si = None if s0 is None else s0.to(DEV)
    zi = None if z0 is None else z0.to(DEV)
    o, den, _, _, saved = la.linattn_forward_train(d[0], d[1], d[2], si, zi, phi=phi)
    o_plain, _, _ = la.linattn_forward(d[0], d[1], d[2], si, zi, phi=phi)
    dq, dk, dv = la.linattn_backward(d[0], d[1], d[2], den, d[3], si, zi, phi=phi,
                                     saved=saved if use_saved else None)
    torch.cuda.synchronize()
    # the same quantity; the training forward sums its segment states in the
    # backward's form, so a few outputs may differ in their last bit
    assert_close("o (training vs plain forward)", o.cpu(), o_plain.cpu(), 1e-2)
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(q, k, v, g, phi=la.PHI_ELU1, s0=None, z0=None, use_saved=True):
    dq, dk, dv = run(q, k, v, g, phi, s0, z0, use_saved)
    rq, rk, rv, _, _ = oracle.backward(q, k, v, g, s0, z0, phi_mode=phi)
    ro, _, _ = oracle.forward(q, k, v, s0, z0, phi_mode=phi)
    tol = TOL[torch.bfloat16]
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert_close(f"{name} heads", got, ref, tol, per="head")
    assert_close("dq rows (floored by the term size)", dq, rq, tol, floor=dq_term_size(q, k, g, ro, s0, z0, phi))
    assert_close("dk rows (floored by the terms' root-sum-square)", dk, rk, tol,
                 floor=dk_term_size(q, k, v, g, ro, s0, z0, phi))
    assert_close("dv rows", dv, rv, tol)


@pytest.mark.parametrize("shape", [(1, 2, 700, 64, 64), (1, 1, 5000, 128, 128), (2, 2, 1000, 64, 128),
                                   (1, 3, 777, 128, 64), (1, 1, 64, 128, 128), (1, 1, 2, 64, 64),
                                   (1, 1, 65, 128, 128), (4, 8, 300, 64, 64), (1, 2, 16385, 128, 128),
                                   (16, 16, 64, 64, 64)])
def test_backward(shape):
    check(*make(*shape, seed=700 + sum(shape)))


@pytest.mark.parametrize("shape", [(1, 2, 700, 64, 64), (1, 1, 5000, 128, 128), (2, 2, 1000, 64, 128),
                                   (1, 3, 777, 128, 64)])
def test_backward_recomputing_the_segment_states(shape):
    # without the training forward's states: the backward's own state pass
    check(*make(*shape, seed=700 + sum(shape)), use_saved=False)


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 128), (64, 128)])
def test_backward_one_token(Dk, Dv):
    # One token: o = v s / (s + eps) with s = phi(q).phi(k), so dq and dk are
    # (v . dY) eps / (s + eps) times phi(k) phi'(q), resp. phi(q) phi'(k):
    # eps-sized differences of terms of size |phi| |v . dY|, against which
    # alone an error bound means anything.  dv is compared as usual.
    q, k, v, g = make(3, 2, 1, Dk, Dv, seed=750 + Dk + Dv)
    dq, dk, dv = run(q, k, v, g)
    rq, rk, rv, _, _ = oracle.backward(q, k, v, g)
    tol = TOL[torch.bfloat16]
    assert_close("dv", dv, rv, tol, per="head")
    q64, k64, v64, g64 = (x.double().numpy() for x in (q, k, v, g))
    fq, fk = oracle.phi(q64), oracle.phi(k64)
    s = (fq * fk).sum(-1)
    vdy = np.abs((v64 * g64).sum(-1)) / (s + 1e-6)  # |v . dY|, [B, H, 1]
    for name, got, ref, f in (("dq", dq, rq, fk), ("dk", dk, rk, fq)):
        terms = np.abs(f).max(-1) * vdy
        err = np.abs(got.double().numpy() - ref).max(-1)
        print(f"  {name}: max |err| / term size {float((err / terms).max()):.3e} (tol {tol:.0e})")
        assert (err <= tol * terms).all(), name


@pytest.mark.parametrize("shape", [(1, 2, 2000, 128, 128), (1, 2, 700, 64, 128)])
def test_backward_unscaled_inputs(shape):
    # q, k drawn N(0, 1) without the 1/sqrt(D) scale: features and denominators
    # over a wider range (phi up to ~e^3, den in the thousands)
    check(*make(*shape, seed=760 + sum(shape), scale=1.0))


@pytest.mark.parametrize("use_saved", [True, False])
def test_backward_identity_map(use_saved):
    check(*make(1, 2, 900, 128, 128, seed=741, positive=True), phi=la.PHI_IDENTITY, use_saved=use_saved)


@pytest.mark.parametrize("use_saved", [True, False])
def test_backward_with_initial_state(use_saved):
    q, k, v, g = make(1, 2, 3000, 128, 128, seed=742)
    gen = torch.Generator().manual_seed(3)
    s0 = torch.randn(1, 2, 128, 128, generator=gen)
    z0 = torch.rand(1, 2, 128, generator=gen) * 50 + 20
    check(q, k, v, g, s0=s0, z0=z0, use_saved=use_saved)


def test_backward_deterministic():
    q, k, v, g = (x.to(DEV) for x in make(1, 4, 9000, 128, 128, seed=743))
    _, den, _, _, saved = la.linattn_forward_train(q, k, v)
    r1 = la.linattn_backward(q, k, v, den, g, saved=saved)
    r2 = la.linattn_backward(q, k, v, den, g, saved=saved)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)
