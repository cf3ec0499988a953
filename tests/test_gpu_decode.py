"""GPU parity of the one-token decode step (in-place update of S and z)."""
import pytest
import torch

import oracle
from linear_attention_phi_amd import binding as la
from linear_attention_phi_amd import synth
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def state_after_prefix(B, H, Dk, Dv, dtype, seed, prefix=256):
    """fp32 (S, z) of a seeded random prefix, built by the oracle (fp64, rounded once)."""
    w = synth.Workload("p", B, H, prefix, Dk, Dv, dtype, seed, q_scale=Dk ** -0.5, k_scale=Dk ** -0.5,
                       v_scale=Dk ** -0.5)
    _, k, v = synth.qkv(w)
    s, z = oracle.state_from_prefix(k, v)
    return torch.from_numpy(s).float().contiguous(), torch.from_numpy(z).float().contiguous()


@pytest.mark.parametrize("B,H,Dk,Dv,dtype", [
    (2, 3, 128, 128, torch.bfloat16), (4, 2, 64, 64, torch.bfloat16), (1, 5, 16, 128, torch.bfloat16),
    (3, 1, 128, 16, torch.bfloat16), (2, 2, 32, 64, torch.float32), (1, 1, 16, 16, torch.float32),
    (2, 4, 128, 128, torch.float32)])
@pytest.mark.parametrize("gated", [False, True])
def test_decode_step(B, H, Dk, Dv, dtype, gated):
    seed = 700 + B + H + Dk + Dv
    s0, z0 = state_after_prefix(B, H, Dk, Dv, dtype, seed)
    w = synth.Workload("d", B, H, 1, Dk, Dv, dtype, seed + 1, q_scale=Dk ** -0.5, k_scale=Dk ** -0.5,
                       v_scale=Dk ** -0.5)
    q, k, v = (x[:, :, 0].contiguous() for x in synth.qkv(w))
    a = synth.gate_heads(seed, B, H, 1)[:, :, 0].contiguous() if gated else None
    sd, zd = s0.to(DEV), z0.to(DEV)
    o = la.linattn_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), sd, zd, None if a is None else a.to(DEV))
    torch.cuda.synchronize()
    ro, rs, rz = oracle.decode_step(q, k, v, s0, z0, alpha=a)
    tol = TOL[dtype]
    assert_close("o", o.cpu(), ro, tol)
    # the state is fp32 whatever the input dtype: one fp32 update from fp32 values
    assert_close("S", sd.cpu(), rs, 1e-5, per="head")
    assert_close("z", zd.cpu(), rz, 1e-5, per="head")


def test_decode_continues_the_forward():
    """decode(forward(prefix).state, token) equals forward(prefix + token)'s last row and state."""
    B, H, N, D = 2, 2, 999, 128
    w = synth.Workload("c", B, H, N + 1, D, D, torch.bfloat16, 710, q_scale=D ** -0.5, k_scale=D ** -0.5)
    q, k, v = (x.to(DEV) for x in synth.qkv(w))
    o_all, s_all, z_all = la.linattn_forward(q, k, v)
    _, s, z = la.linattn_forward(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(), v[:, :, :N].contiguous())
    od = la.linattn_decode_step(q[:, :, N].contiguous(), k[:, :, N].contiguous(), v[:, :, N].contiguous(), s, z)
    torch.cuda.synchronize()
    # the forward rounds phi(k) to bf16 for the matrix cores, the decode step
    # keeps it in fp32: the two agree to the bf16 tolerance
    tol = TOL[torch.bfloat16]
    assert_close("o", od.cpu(), o_all[:, :, N].cpu(), tol)
    assert_close("S", s.cpu(), s_all.cpu(), tol, per="head")
    assert_close("z", z.cpu(), z_all.cpu(), tol, per="head")


def test_decode_steps_reproduce_worked_states():
    from conftest import golden
    g = golden("fixed_size_state_2x2.json")
    s = torch.zeros(1, 1, 16, 16, device=DEV)
    z = torch.zeros(1, 1, 16, device=DEV)
    for t in range(3):
        def row(x):
            r = torch.zeros(1, 1, 16)
            r[0, 0, :2] = torch.tensor(x, dtype=torch.float32)
            return r.to(DEV)
        o = la.linattn_decode_step(row(g["q"][t]), row(g["k"][t]), row(g["v"][t]), s, z, eps=0.0,
                                   phi=la.PHI_IDENTITY)
        torch.cuda.synchronize()
        assert s.cpu()[0, 0, :2, :2].tolist() == g["printed"]["state_after_token"][t]
        assert torch.allclose(o.cpu()[0, 0, :2], torch.tensor(g["derived"]["y"][t], dtype=torch.float32))
