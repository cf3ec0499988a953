"""GPU parity on the five measured workloads at full size, in the launch
configuration the benchmark times, and on the backward as the benchmark times
it (over the 131072-token workload).

On the 131072-token workload the forward's outputs are compared on every row
of every head; its backward and snapshot forwards on four heads spread over
the sixteen (every gradient row, every snapshot position); elsewhere every
output is checked.
"""
import time

import numpy as np
import pytest
import torch

import oracle
from linear_attention_phi_amd import binding as la
from linear_attention_phi_amd import synth
from parity import TOL, assert_close, dk_term_size, dq_term_size

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def stamp(msg):
    print(f"  [{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def test_tiny_fp32():
    w = synth.WORKLOADS["tiny_fp32"]
    q, k, v = synth.qkv(w)
    o, s, z = la.linattn_forward(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    ro, rs, rz = oracle.forward(q, k, v)
    assert_close("O", o.cpu(), ro, TOL[w.dtype])
    assert_close("S", s.cpu(), rs, TOL[w.dtype], per="head")
    assert_close("z", z.cpu(), rz, TOL[w.dtype], per="head")
    # the quadratic masked form agrees too
    assert_close("O vs quadratic", o.cpu(), oracle.quadratic_forward(q.double().numpy(), k.double().numpy(),
                                                                      v.double().numpy()), TOL[w.dtype])


def test_b4h8_n4096_d64():
    w = synth.WORKLOADS["b4h8_n4096_d64"]
    q, k, v = synth.qkv(w)
    o, s, z = la.linattn_forward(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    ro, rs, rz = oracle.forward(q, k, v)
    assert_close("O", o.cpu(), ro, TOL[w.dtype])
    assert_close("S", s.cpu(), rs, TOL[w.dtype], per="head")
    assert_close("z", z.cpu(), rz, TOL[w.dtype], per="head")


def test_long_n131072_d128_sampled():
    w = synth.WORKLOADS["long_n131072_d128"]
    stamp("generating inputs")
    q, k, v = synth.qkv(w)
    stamp("GPU forward")
    o, s, z = la.linattn_forward(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    o, s, z = o.cpu(), s.cpu(), z.cpu()
    assert torch.isfinite(o.float()).all()
    stamp("oracle: final state of every head (library contraction)")
    rs, rz = oracle.state_from_prefix(k[0], v[0])
    assert_close("S (all heads)", s, rs[None], TOL[w.dtype], per="head")
    assert_close("z (all heads)", z, rz[None], TOL[w.dtype], per="head")
    stamp(f"oracle: all {w.H} heads, all {w.N} rows")
    ro, rsh, _ = oracle.forward(q, k, v)
    assert_close("O (all heads)", o, ro, TOL[w.dtype])
    assert_close("S (all heads, recurrence)", s, rsh, TOL[w.dtype], per="head")


SPREAD_HEADS = [0, 5, 10, 15]


def test_backward_on_the_long_workload_sampled():
    # the backward as the benchmark times it (all 16 heads of the 131072-token
    # workload in one call, dO seeded N(0, 1)); the gradients of the first and
    # last head against the oracle's adjoint recurrence
    w = synth.WORKLOADS["long_n131072_d128"]
    stamp("generating inputs")
    q, k, v = synth.qkv(w)
    g = synth.dout(w)
    stamp("GPU training forward and backward")
    d = [x.to(DEV) for x in (q, k, v, g)]
    _, den, _, _, saved = la.linattn_forward_train(d[0], d[1], d[2])
    dq, dk, dv = la.linattn_backward(d[0], d[1], d[2], den, d[3], saved=saved)
    torch.cuda.synchronize()
    hs = SPREAD_HEADS
    got = [x[:, hs].cpu() for x in (dq, dk, dv)]
    del d, den, saved, dq, dk, dv
    stamp(f"oracle: gradients of heads {hs}")
    qh, kh, vh, gh = (x[:, hs] for x in (q, k, v, g))
    rq, rk, rv, _, _ = oracle.backward(qh, kh, vh, gh)
    ro, _, _ = oracle.forward(qh, kh, vh)
    stamp("term sizes of the cancelling rows (dq, dk)")
    floors = {"dq": dq_term_size(qh, kh, gh, ro), "dk": dk_term_size(qh, kh, vh, gh, ro), "dv": None}
    for name, x, r in zip(("dq", "dk", "dv"), got, (rq, rk, rv)):
        assert torch.isfinite(x.float()).all()
        assert_close(f"{name} heads {hs}", x, r, TOL[w.dtype], per="head")
        assert_close(f"{name} rows, heads {hs}", x, r, TOL[w.dtype], floor=floors[name])


def test_snapshots_on_the_long_workload_sampled():
    # the snapshot forward as the benchmark times it: 8 prefix-cache points at
    # 16384 m - 1 and the last 8 tokens of the 131072-token workload; the states
    # of four spread heads at every position against the prefix sum
    w = synth.WORKLOADS["long_n131072_d128"]
    stamp("generating inputs")
    q, k, v = synth.qkv(w)
    pos = sorted({16384 * m - 1 for m in range(1, 9) if 16384 * m - 1 < w.N} | {w.N - 1 - i for i in range(8)})
    stamp("GPU forward with snapshots")
    d = [x.to(DEV) for x in (q, k, v)]
    o, ss, zs, sf, zf = la.linattn_forward_snapshots(*d, pos)
    o2, _, _ = la.linattn_forward(*d)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    hs = SPREAD_HEADS
    ss, zs = ss[:, hs].cpu(), zs[:, hs].cpu()
    del d, o, o2
    stamp(f"oracle: heads {hs} at {len(pos)} positions")
    for i, p in enumerate(pos):
        rs, rz = oracle.state_from_prefix(k[0, hs, :p + 1], v[0, hs, :p + 1])
        assert_close(f"S after token {p}", ss[:, :, i], rs[None], TOL[w.dtype], per="head")
        assert_close(f"z after token {p}", zs[:, :, i], rz[None], TOL[w.dtype], per="head")


def test_gated_b2h16_n16384_d128():
    w = synth.WORKLOADS["gated_b2h16_n16384_d128"]
    q, k, v = synth.qkv(w)
    a = synth.alpha(w)
    o, s, z = la.linattn_forward_gated(q.to(DEV), k.to(DEV), v.to(DEV), a.to(DEV))
    torch.cuda.synchronize()
    stamp("oracle, all heads")
    ro, rs, rz = oracle.forward(q, k, v, alpha=a)
    assert_close("O", o.cpu(), ro, TOL[w.dtype])
    assert_close("S", s.cpu(), rs, TOL[w.dtype], per="head")
    assert_close("z", z.cpu(), rz, TOL[w.dtype], per="head")


def test_decode_b256h32_d128():
    w = synth.WORKLOADS["decode_b256h32_d128"]
    stamp("prefix states (oracle, fp64, rounded once to fp32)")
    s0 = np.empty((w.B, w.H, w.Dk, w.Dv), dtype=np.float32)
    z0 = np.empty((w.B, w.H, w.Dk), dtype=np.float32)
    for b in range(w.B):
        kp, vp = synth.decode_prefix(w, b)
        sb, zb = oracle.state_from_prefix(kp, vp)
        s0[b] = sb
        z0[b] = zb
    s0, z0 = torch.from_numpy(s0), torch.from_numpy(z0)
    q, k, v = synth.decode_token(w)
    sd, zd = s0.to(DEV), z0.to(DEV)
    stamp("GPU decode step")
    o = la.linattn_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), sd, zd)
    torch.cuda.synchronize()
    ro, rs, rz = oracle.decode_step(q, k, v, s0, z0)
    assert_close("o", o.cpu(), ro, TOL[w.dtype])
    assert_close("S", sd.cpu(), rs, 1e-5, per="head")
    assert_close("z", zd.cpu(), rz, 1e-5, per="head")


def test_noncausal_on_the_long_workload_sampled():
    w = synth.WORKLOADS["long_n131072_d128"]
    hs = [3, 12]
    q, k, v = synth.qkv(w)
    o, s, z = la.linattn_forward_noncausal(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    o, s = o.cpu(), s.cpu()
    rs, rz = oracle.state_from_prefix(k[0], v[0])
    assert_close("S (all heads)", s, rs[None], TOL[w.dtype], per="head")
    ro, _, _ = oracle.noncausal(q[:, hs], k[:, hs], v[:, hs])
    assert_close(f"O heads {hs}", o[:, hs], ro, TOL[w.dtype])
