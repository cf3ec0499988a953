"""linattn_forward_noalloc against linattn_forward, through the C ABI.

The no-allocation forward runs the same kernels with the same segment plan as
linattn_forward; only the segment states live in the library's fixed device
scratch instead of the caller's workspace.  So its outputs must equal
linattn_forward's bit for bit.  Three calls in a row share the one scratch:
the 131072-token, 16-head workload (35 MB of segment states) on the null
stream; a smaller, ragged input with a different plan on a side stream (the
scratch then holds the first call's stale states, which must not matter);
and the first input again.
"""
import pytest
import torch

from linear_attention_phi_amd import binding as la
from linear_attention_phi_amd import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def inputs(B, H, N, D, seed):
    w = synth.Workload("t", B, H, N, D, D, torch.bfloat16, seed, q_scale=D ** -0.5, k_scale=D ** -0.5,
                       v_scale=D ** -0.5)
    return [x.to(DEV) for x in synth.qkv(w)]


def outputs_like(q, v):
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    return (torch.empty((B, H, N, Dv), dtype=q.dtype, device=DEV),
            torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=DEV),
            torch.empty((B, H, Dk), dtype=torch.float32, device=DEV))


def noalloc(q, k, v, s0=None, z0=None):
    o, s, z = outputs_like(q, v)
    la.linattn_forward_noalloc(q, k, v, s0, z0, out=o, s_final=s, z_final=z)
    return o, s, z


def assert_same(a, b):
    for x, y, name in zip(a, b, ("o", "s_final", "z_final")):
        assert torch.equal(x, y), name


def test_noalloc_forward_equals_the_workspace_forward_on_consecutive_calls():
    big = inputs(1, 16, 131072, 128, seed=2201)
    small = inputs(2, 3, 5000, 64, seed=2202)
    assert la.workspace_size(la.KIND_FORWARD, 1, 16, 131072, 128, 128, la.BF16) > \
        la.workspace_size(la.KIND_FORWARD, 2, 3, 5000, 64, 64, la.BF16) > 0

    first = noalloc(*big)
    ref_big = la.linattn_forward(*big)
    torch.cuda.synchronize()
    assert_same(first, ref_big)

    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        second = noalloc(*small)
        ref_small = la.linattn_forward(*small)
    torch.cuda.synchronize()
    assert_same(second, ref_small)

    third = noalloc(*big)
    torch.cuda.synchronize()
    assert_same(third, first)


def test_noalloc_forward_resumes_from_an_initial_state():
    q, k, v = inputs(1, 4, 20000, 128, seed=2203)
    h = 12000
    o1, s1, z1 = noalloc(q[:, :, :h].contiguous(), k[:, :, :h].contiguous(), v[:, :, :h].contiguous())
    o2, s2, z2 = noalloc(q[:, :, h:].contiguous(), k[:, :, h:].contiguous(), v[:, :, h:].contiguous(), s1, z1)
    r2 = la.linattn_forward(q[:, :, h:].contiguous(), k[:, :, h:].contiguous(), v[:, :, h:].contiguous(), s1, z1)
    torch.cuda.synchronize()
    assert_same((o2, s2, z2), r2)
