"""GPU parity of the delta rule against the fp64 oracle.

linattn_forward_delta runs through the C ABI; O is compared row-normwise and
the final state per head with oracle.delta on the same seeded bf16 inputs
(q, k, v drawn N(0, 1): with elu + 1 the unit keys are then far from all
parallel).  Shapes span several chunks, ragged tails, one token, both head
dims and their mix; beta absent (full overwrite) or drawn in (0, 1); an
initial state; the gated form (gates sigmoid(N(4, 1)) with an exact zero, and
gates of one against the ungated kernel); and the product-order page's worked
example (keys in two of 64 dims, the identity map) on the GPU path.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from linear_attention_phi_amd import binding as la
from linear_attention_phi_amd import synth
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF = torch.bfloat16


def make(B, H, N, Dk, Dv, seed, with_beta=False):
    w = synth.Workload("t", B, H, N, Dk, Dv, BF, seed)
    q, k, v = synth.qkv(w)
    beta = None
    if with_beta:
        beta = torch.sigmoid(synth.normal_heads(seed, synth.G_ID, B, H, N, 1, 1.0, torch.float32)[..., 0])
    return q, k, v, beta


def check(q, k, v, beta=None, s0=None, phi=la.PHI_ELU1, alpha=None):
    d = [x.to(DEV) for x in (q, k, v)]
    o, s = la.linattn_forward_delta(*d, None if beta is None else beta.to(DEV),
                                    None if s0 is None else s0.to(DEV), phi=phi,
                                    alpha=None if alpha is None else alpha.to(DEV))
    torch.cuda.synchronize()
    ro, rs = oracle.delta(q, k, v, beta, s0, alpha=alpha, phi_mode=phi)
    tol = TOL[BF]
    assert_close("O", o.cpu(), ro, tol)
    assert_close("S", s.cpu(), rs, tol, per="head")
    return o, s


@pytest.mark.parametrize("shape", [(1, 2, 700, 64, 64), (2, 2, 1000, 128, 128), (1, 3, 333, 64, 128),
                                   (1, 1, 1, 128, 128), (1, 1, 65, 128, 64), (4, 4, 200, 128, 128)])
def test_delta(shape):
    check(*make(*shape, seed=1200 + sum(shape)))


def test_delta_full_length():
    # the delta workload's length and head dims (64 chunks), two of its heads,
    # its seed and unscaled inputs: the error of a long chunk chain
    w = synth.WORKLOADS["delta_b16h16_n4096_d128"]
    x = synth.Workload("t", 1, 2, w.N, w.Dk, w.Dv, BF, w.seed)
    check(*synth.qkv(x))


def test_gated_delta_full_length():
    # the workload's length (64 chunks) with gates a = sigmoid(N(4, 1)), beta and
    # an initial state: the gated chain over every chunk
    w = synth.WORKLOADS["delta_b16h16_n4096_d128"]
    q, k, v, beta = make(1, 2, w.N, w.Dk, w.Dv, seed=w.seed + 1, with_beta=True)
    a = synth.gate_heads(1280, 1, 2, w.N)
    s0 = torch.randn(1, 2, w.Dk, w.Dv, generator=torch.Generator().manual_seed(14)) * 0.1
    check(q, k, v, beta, s0, alpha=a)


@pytest.mark.parametrize("shape", [(1, 2, 700, 128, 128), (2, 1, 130, 64, 64), (1, 2, 333, 128, 64),
                                   (1, 1, 64, 64, 128)])
def test_delta_with_beta(shape):
    check(*make(*shape, seed=1220 + sum(shape), with_beta=True))


def test_delta_with_initial_state_and_resume():
    q, k, v, beta = make(1, 2, 600, 128, 128, seed=1230, with_beta=True)
    s0 = torch.randn(1, 2, 128, 128, generator=torch.Generator().manual_seed(7)) * 0.1
    o, s = check(q, k, v, beta, s0)
    # two calls (the second from the first's final state) give the same tail
    o1, s1 = la.linattn_forward_delta(q[:, :, :256].to(DEV), k[:, :, :256].to(DEV), v[:, :, :256].to(DEV),
                                      beta[:, :, :256].to(DEV), s0.to(DEV))
    o2, s2 = la.linattn_forward_delta(q[:, :, 256:].to(DEV), k[:, :, 256:].to(DEV), v[:, :, 256:].to(DEV),
                                      beta[:, :, 256:].to(DEV), s1)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu(), o[:, :, 256:].cpu()) and torch.equal(s2.cpu(), s.cpu())


@pytest.mark.parametrize("shape", [(1, 2, 700, 128, 128), (2, 2, 333, 64, 128), (1, 1, 65, 128, 64)])
def test_gated_delta(shape):
    # gates a = sigmoid(N(4, 1)) (a memory of ~50 tokens), one exact zero gate
    q, k, v, beta = make(*shape, seed=1240 + sum(shape), with_beta=True)
    a = synth.gate_heads(1240 + sum(shape), *shape[:3])
    a[0, 0, shape[2] // 2] = 0.0
    s0 = torch.randn(*shape[:2], shape[3], shape[4], generator=torch.Generator().manual_seed(9)) * 0.1
    check(q, k, v, beta, s0, alpha=a)
    check(q, k, v, alpha=a)


def test_gate_of_one_equals_ungated_on_the_gpu():
    q, k, v, _ = make(1, 2, 200, 128, 128, seed=1250)
    d = [x.to(DEV) for x in (q, k, v)]
    o1, s1 = la.linattn_forward_delta(*d)
    o2, s2 = la.linattn_forward_delta(*d, alpha=torch.ones(1, 2, 200, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("shape", [(1, 2, 300, 128, 128), (1, 1, 200, 64, 128), (1, 2, 150, 64, 64)])
def test_delta_identity_map(shape):
    # the identity feature map (keys normalized as they are, negative entries
    # included) through both kernels and both gate forms
    q, k, v, beta = make(*shape, seed=1260 + sum(shape), with_beta=True)
    check(q, k, v, beta, phi=la.PHI_IDENTITY)
    a = synth.gate_heads(1260 + sum(shape), *shape[:3])
    check(q, k, v, beta, phi=la.PHI_IDENTITY, alpha=a)


@pytest.mark.parametrize("shape", [(1, 2, 300, 128, 128), (2, 1, 200, 128, 64)])
def test_delta_final_state_in_place(shape):
    # through the C ABI with s_final at s_init's address (the header allows it):
    # the same outputs and state as with separate buffers, both kernels
    q, k, v, beta = make(*shape, seed=1270 + sum(shape), with_beta=True)
    B, H, N, Dk, Dv = shape
    d = [x.to(DEV) for x in (q, k, v, beta)]
    s0 = (torch.randn(B, H, Dk, Dv, generator=torch.Generator().manual_seed(11)) * 0.1).to(DEV)
    o1, s1 = la.linattn_forward_delta(d[0], d[1], d[2], d[3], s0.clone())
    s = s0.clone()
    o2 = torch.empty_like(o1)
    rc = la.lib().linattn_forward_delta(la._ptr(d[0]), la._ptr(d[1]), la._ptr(d[2]), None, la._ptr(d[3]),
                                        la._ptr(o2), la._ptr(s), la._ptr(s), B, H, N, Dk, Dv, la.BF16,
                                        la.PHI_ELU1, la._stream(d[0]))
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s)


def test_worked_example_on_the_gpu():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "summary_scalar_values.json")))
    D = 64
    keys = np.zeros((3, D))
    keys[:, :2] = g["keys"]
    vals = np.zeros((3, D))
    vals[:, 0] = g["values"]
    qs = keys.copy()
    qs[2] = 0.0
    qs[2, 0] = 1.0  # the last read uses the query (1, 0)
    q, k, v = (torch.tensor(x[None, None], dtype=BF) for x in (qs, keys, vals))
    o, s = check(q, k, v, phi=la.PHI_IDENTITY)
    p = g["printed"]["delta_rule"]
    # bf16 inputs (0.6 and 0.8 are not exact in bf16) and bf16 operands: within 1%
    np.testing.assert_allclose(s[0, 0, :2, 0].cpu().numpy(), p["state"], rtol=1e-2)
    np.testing.assert_allclose(float(o[0, 0, 2, 0]), p["read_with_1_0"], rtol=1e-2)
