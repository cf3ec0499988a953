"""GPU parity of the state snapshots (the summary after chosen tokens).

linattn_forward_snapshots runs through the C ABI; its o and final state must
equal the plain forward's bit for bit (same kernels), and every snapshot is
compared on its own, normwise per (b, h, position), with oracle.snapshots on
the same seeded inputs (z grows with the position, so one early snapshot must
not be judged against the size of a later one).  Positions
sit on and next to chunk (64) and state-cell boundaries, at the first and
last token, repeated and out of order; the one-segment plan (many heads) runs
every snapshot from the initial state.
"""
import pytest
import torch

import oracle
from linear_attention_phi_amd import binding as la
from linear_attention_phi_amd import synth
from parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def make(B, H, N, Dk, Dv, seed, gated=False):
    w = synth.Workload("t", B, H, N, Dk, Dv, torch.bfloat16, seed, q_scale=Dk ** -0.5, k_scale=Dk ** -0.5)
    q, k, v = synth.qkv(w)
    a = synth.gate_heads(seed, B, H, N) if gated else None
    return q, k, v, a


def check(q, k, v, positions, a=None, s0=None, z0=None):
    d = [x.to(DEV) for x in (q, k, v)]
    ad = None if a is None else a.to(DEV)
    si = None if s0 is None else s0.to(DEV)
    zi = None if z0 is None else z0.to(DEV)
    o, ss, zs, sf, zf = la.linattn_forward_snapshots(*d, positions, ad, si, zi)
    if ad is None:
        o2, sf2, zf2 = la.linattn_forward(*d, si, zi)
    else:
        o2, sf2, zf2 = la.linattn_forward_gated(*d, ad, si, zi)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(sf, sf2) and torch.equal(zf, zf2)
    rs, rz = oracle.snapshots(q, k, v, positions, s0, z0, alpha=a)
    tol = TOL[torch.bfloat16]
    assert_close("S snapshots", ss.cpu(), rs, tol, per="item")
    assert_close("z snapshots", zs.cpu(), rz, tol, per="item")
    return ss, zs, sf, zf


@pytest.mark.parametrize("shape", [(1, 2, 6000, 128, 128), (1, 3, 3000, 64, 128), (2, 1, 3000, 128, 64)])
def test_snapshots(shape):
    # few heads: many segments, state cells of one or a few chunks
    q, k, v, _ = make(*shape, seed=1100 + sum(shape))
    N = shape[2]
    check(q, k, v, [N // 2, 0, 63, 64, 65, 191, 192, N - 1, N // 2])


def test_snapshots_in_a_long_last_segment():
    # 64 heads of 2048 tokens: 4 segments of 512 tokens and cells of 256; the
    # last segment has no cells of its own, so its snapshots run from 1536
    q, k, v, _ = make(4, 16, 2048, 64, 64, seed=1110)
    check(q, k, v, [1535, 1536, 2047, 100])


def test_snapshots_gated_with_zero_gate():
    q, k, v, a = make(1, 2, 6000, 128, 128, seed=1120, gated=True)
    a[0, 1, 3000] = 0.0
    check(q, k, v, [0, 2999, 3000, 3001, 4095, 4096, 5999], a)


def test_snapshots_with_initial_state_and_one_segment():
    # 256 heads: the plan has one segment per head, so snapshots start from the initial state
    q, k, v, _ = make(16, 16, 100, 64, 64, seed=1130)
    gen = torch.Generator().manual_seed(5)
    s0 = torch.randn(16, 16, 64, 64, generator=gen)
    z0 = torch.rand(16, 16, 64, generator=gen) * 10 + 5
    check(q, k, v, [0, 50, 63, 64, 99], s0=s0, z0=z0)


def test_last_snapshot_is_the_final_state():
    q, k, v, _ = make(1, 2, 10000, 128, 128, seed=1140)
    ss, zs, sf, zf = check(q, k, v, [9999])
    # same sums in a different order (cell prefix + range vs the output pass's carry)
    assert_close("S final", ss[:, :, 0].cpu(), sf.cpu().double().numpy(), 1e-5, per="head")
    assert_close("z final", zs[:, :, 0].cpu(), zf.cpu().double().numpy(), 1e-5, per="head")
