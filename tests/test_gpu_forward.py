"""GPU parity of the causal forward (plain and gated) and the non-causal form.

Every case runs the HIP library through the C ABI and compares element by
element with the fp64 oracle on the same seeded inputs, at sizes that span
several chunks, several segments per head and a ragged tail.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import golden
from linear_attention_phi_amd import binding as la
from linear_attention_phi_amd import synth
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def make(B, H, N, Dk, Dv, dtype, seed, gated=False):
    w = synth.Workload("t", B, H, N, Dk, Dv, dtype, seed, q_scale=Dk ** -0.5, k_scale=Dk ** -0.5)
    q, k, v = synth.qkv(w)
    a = synth.gate_heads(seed, B, H, N) if gated else None
    return q, k, v, a


def run_and_check(q, k, v, a, tol, eps=1e-6, s_init=None, z_init=None, phi=la.PHI_ELU1):
    args = [x.to(DEV) for x in (q, k, v)]
    si = None if s_init is None else s_init.to(DEV)
    zi = None if z_init is None else z_init.to(DEV)
    if a is None:
        o, s, z = la.linattn_forward(*args, si, zi, eps=eps, phi=phi)
    else:
        o, s, z = la.linattn_forward_gated(*args, a.to(DEV), si, zi, eps=eps, phi=phi)
    torch.cuda.synchronize()
    ro, rs, rz = oracle.forward(q, k, v, s_init, z_init, alpha=a, eps=eps, phi_mode=phi)
    assert_close("O", o.cpu(), ro, tol)
    assert_close("S", s.cpu(), rs, tol, per="head")
    assert_close("z", z.cpu(), rz, tol, per="head")
    return o, s, z


BF16_SHAPES = [
    (1, 2, 700, 64, 64), (2, 3, 1, 32, 32), (1, 1, 63, 128, 128), (1, 1, 64, 128, 128), (1, 1, 65, 128, 128),
    (2, 2, 1000, 32, 128), (1, 3, 777, 128, 64), (1, 1, 5000, 128, 128), (4, 8, 300, 64, 64), (1, 2, 4096, 64, 32),
    (3, 1, 2500, 128, 32),
]
F32_SHAPES = [
    (1, 1, 64, 16, 16), (1, 2, 300, 32, 32), (2, 1, 1000, 64, 64), (1, 1, 129, 128, 128), (1, 1, 2000, 16, 64),
    (1, 1, 1, 16, 16),
]
BF16_VALU_SHAPES = [(1, 2, 500, 16, 16), (1, 1, 300, 16, 64), (1, 1, 200, 64, 16)]


@pytest.mark.parametrize("shape", BF16_SHAPES + BF16_VALU_SHAPES)
def test_forward_bf16(shape):
    q, k, v, _ = make(*shape, torch.bfloat16, seed=100 + sum(shape))
    run_and_check(q, k, v, None, TOL[torch.bfloat16])


@pytest.mark.parametrize("shape", F32_SHAPES)
def test_forward_fp32(shape):
    q, k, v, _ = make(*shape, torch.float32, seed=200 + sum(shape))
    run_and_check(q, k, v, None, TOL[torch.float32])


@pytest.mark.parametrize("shape", [(1, 2, 700, 64, 64), (1, 1, 5000, 128, 128), (2, 2, 1000, 32, 128),
                                   (1, 3, 777, 128, 64), (1, 2, 500, 16, 16)])
def test_gated_bf16(shape):
    q, k, v, a = make(*shape, torch.bfloat16, seed=300 + sum(shape), gated=True)
    run_and_check(q, k, v, a, TOL[torch.bfloat16])


@pytest.mark.parametrize("shape", [(1, 1, 64, 16, 16), (1, 2, 1000, 32, 32), (1, 1, 300, 128, 64)])
def test_gated_fp32(shape):
    q, k, v, a = make(*shape, torch.float32, seed=400 + sum(shape), gated=True)
    run_and_check(q, k, v, a, TOL[torch.float32])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gated_strong_decay_and_exact_zeros(dtype):
    B, H, N, D = 1, 2, 3000, 64
    q, k, v, _ = make(B, H, N, D, D, dtype, seed=501)
    g = torch.Generator().manual_seed(5)
    a = torch.rand(B, H, N, generator=g) * 0.9 + 0.05
    a[0, 0, 100] = 0.0          # clears the summary mid-chunk
    a[0, 1, 64 * 10] = 0.0      # at a chunk boundary
    a[0, 1, 2047] = 0.0
    run_and_check(q, k, v, a, TOL[dtype])


def test_gate_of_one_is_bitwise_ungated():
    q, k, v, _ = make(1, 2, 3000, 128, 128, torch.bfloat16, seed=502)
    args = [x.to(DEV) for x in (q, k, v)]
    o1, s1, z1 = la.linattn_forward(*args)
    o2, s2, z2 = la.linattn_forward_gated(*args, torch.ones(1, 2, 3000, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(z1, z2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_resume_from_state(dtype):
    q, k, v, _ = make(2, 2, 1500, 64, 64, dtype, seed=503)
    n1 = 700
    args1 = [x[:, :, :n1].contiguous().to(DEV) for x in (q, k, v)]
    args2 = [x[:, :, n1:].contiguous().to(DEV) for x in (q, k, v)]
    o1, s1, z1 = la.linattn_forward(*args1)
    o2, s2, z2 = la.linattn_forward(*args2, s1, z1)
    torch.cuda.synchronize()
    ro, rs, rz = oracle.forward(q, k, v)
    tol = TOL[dtype]
    assert_close("O", torch.cat([o1, o2], dim=2).cpu(), ro, tol)
    assert_close("S", s2.cpu(), rs, tol, per="head")
    # in place: s_final aliasing s_init
    s_in, z_in = s1.clone(), z1.clone()
    la.linattn_forward(*args2, s_in, z_in, s_final=s_in, z_final=z_in)
    torch.cuda.synchronize()
    assert torch.equal(s_in, s2) and torch.equal(z_in, z2)


def test_initial_state_is_used_gated():
    q, k, v, a = make(1, 2, 2000, 128, 128, torch.bfloat16, seed=504, gated=True)
    g = torch.Generator().manual_seed(9)
    s0 = torch.randn(1, 2, 128, 128, generator=g) * 4
    z0 = torch.rand(1, 2, 128, generator=g) * 500 + 100
    run_and_check(q, k, v, a, TOL[torch.bfloat16], s_init=s0, z_init=z0)


def test_deterministic_bitwise():
    q, k, v, a = make(1, 4, 8000, 128, 128, torch.bfloat16, seed=505, gated=True)
    args = [x.to(DEV) for x in (q, k, v)]
    ad = a.to(DEV)
    r1 = la.linattn_forward_gated(*args, ad)
    r2 = la.linattn_forward_gated(*args, ad)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def _pad(rows, D=16):
    x = np.zeros((1, 1, len(rows), D))
    for t, r in enumerate(rows):
        x[0, 0, t, :len(r)] = r
    return torch.from_numpy(x).float()


def test_worked_example_through_the_gpu():
    g = golden("fixed_size_state_2x2.json")
    q, k, v = _pad(g["q"]), _pad(g["k"]), _pad(g["v"])
    o, s, z = la.linattn_forward(q.to(DEV), k.to(DEV), v.to(DEV), eps=0.0, phi=la.PHI_IDENTITY)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s.cpu()[0, 0, :2, :2].numpy(), g["printed"]["state_after_token"][2])
    np.testing.assert_array_equal(z.cpu()[0, 0, :2].numpy(), g["printed"]["z_final"])
    np.testing.assert_allclose(o.cpu()[0, 0, :, :2].numpy(), g["derived"]["y"], atol=1e-7)
    on, sn, zn = la.linattn_forward_noncausal(q.to(DEV), k.to(DEV), v.to(DEV), eps=0.0, phi=la.PHI_IDENTITY)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sn.cpu()[0, 0, :2, :2].numpy(), g["printed"]["noncausal_state"])
    np.testing.assert_allclose(on.cpu()[0, 0, :, :2].numpy(), g["derived"]["noncausal_y"], atol=1e-7)


def test_scalar_example_through_the_gpu():
    g = golden("summary_scalar_values.json")
    keys = _pad(g["keys"])
    vals = _pad([[x] for x in g["values"]])
    o, s, z = la.linattn_forward(keys.to(DEV), keys.to(DEV), vals.to(DEV), eps=0.0, phi=la.PHI_IDENTITY)
    torch.cuda.synchronize()
    np.testing.assert_allclose(s.cpu()[0, 0, :2, 0].numpy(), g["printed"]["state_after_three"], rtol=1e-6)
    np.testing.assert_allclose(o.cpu()[0, 0, :, 0].numpy(), g["derived"]["o"], rtol=1e-6)


@pytest.mark.parametrize("shape,dtype", [((1, 2, 700, 64, 64), torch.bfloat16), ((2, 1, 5000, 128, 128), torch.bfloat16),
                                         ((1, 1, 333, 32, 128), torch.bfloat16), ((1, 2, 500, 16, 16), torch.bfloat16),
                                         ((1, 1, 64, 16, 16), torch.float32), ((1, 2, 1000, 64, 32), torch.float32)])
def test_noncausal(shape, dtype):
    q, k, v, _ = make(*shape, dtype, seed=600 + sum(shape))
    o, s, z = la.linattn_forward_noncausal(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    ro, rs, rz = oracle.noncausal(q, k, v)
    tol = TOL[dtype]
    assert_close("O", o.cpu(), ro, tol)
    assert_close("S", s.cpu(), rs, tol, per="head")
    assert_close("z", z.cpu(), rz, tol, per="head")
    # the global state equals the causal final state
    _, sc, zc = la.linattn_forward(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert_close("S vs causal", s.cpu(), sc.cpu(), tol, per="head")


# ---- independence from the split of the sequence (the fixed-size-state page,
# "Adding to the same state in turn": the state is the sum of the outer
# products, whatever way the tokens are grouped).  One input, run with one
# sequential pass, with 16 and with 256 parallel segments (one chunk each):
# every plan within tolerance of the oracle, and the plans within rounding of
# one another.

PLANS = [(1, 1), (16, 2), (256, 1)]


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("D", [128, 64])
def test_results_do_not_depend_on_the_segment_plan(gated, D):
    q, k, v, a = make(1, 2, 256 * 64 - 37, D, D, torch.bfloat16, seed=130 + D + gated, gated=gated)
    args = [x.to(DEV) for x in (q, k, v)]
    ad = None if a is None else a.to(DEV)
    runs = {}
    for P, R in PLANS:
        runs[(P, R)] = [x.cpu() for x in la.linattn_forward_planned(*args, P, R, alpha=ad)]
    torch.cuda.synchronize()
    ro, rs, rz = oracle.forward(q, k, v, alpha=a)
    tol = TOL[torch.bfloat16]
    for plan, (o, s, z) in runs.items():
        assert_close(f"O, plan {plan}", o, ro, tol)
        assert_close(f"S, plan {plan}", s, rs, tol, per="head")
        assert_close(f"z, plan {plan}", z, rz, tol, per="head")
    # the fp32 states differ only by the order of their additions; the bf16
    # outputs by that and a last-bit rounding
    o0, s0, z0 = runs[PLANS[0]]
    for plan in PLANS[1:]:
        o, s, z = runs[plan]
        assert_close(f"O, plan {plan} vs {PLANS[0]}", o, o0, 1e-2)
        assert_close(f"S, plan {plan} vs {PLANS[0]}", s, s0, 1e-5, per="head")
        assert_close(f"z, plan {plan} vs {PLANS[0]}", z, z0, 1e-5, per="head")


def test_default_plan_is_one_of_the_planned_ones():
    # B1 H2 N16384: the library picks 128 segments of 2 chunks, one state part each chunk
    q, k, v, _ = make(1, 2, 16384, 128, 128, torch.bfloat16, seed=140)
    args = [x.to(DEV) for x in (q, k, v)]
    o1, s1, z1 = la.linattn_forward(*args)
    o2, s2, z2 = la.linattn_forward_planned(*args, 128, 2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(z1, z2)
