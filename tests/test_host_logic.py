"""Host-side logic that needs no GPU: flop/byte conventions and the input recipe."""
import math

import numpy as np
import pytest
import torch

from conftest import golden
from linear_attention_phi_amd import roofline, synth


def test_flop_convention_reproduces_the_pages_table():
    t = golden("ssm_tables.json")["flop_table"]
    for n, att, lin, ratio in zip(t["N"], t["attention_flops"], t["linear_flops"], t["ratio"]):
        a = roofline.quadratic_form_flops(n, 64)
        r = roofline.recurrence_flops(n, 64)
        # the page prints rounded millions ("8.4 M", "134 M", "2,147 M")
        assert abs(a - att) / att < 0.01
        assert abs(r - lin) / lin < 0.02
        assert a // r == ratio


def test_long_context_sizes():
    # n = 131072, d = 128: ~1.7e10 score entries vs a 16,384-entry state, ratio 2^20
    n, d = 131072, 128
    assert abs(n * n - 1.7e10) / 1.7e10 < 0.02
    assert d * d == 16384 and (n * n) // (d * d) == 2 ** 20


def test_algorithmic_bytes_of_the_headline_workload():
    w = synth.WORKLOADS["long_n131072_d128"]
    b = roofline.forward_bytes(w.B, w.H, w.N, w.Dk, w.Dv, 2)
    # 3 bf16 inputs + 1 bf16 output per token per head, plus the fp32 final state
    assert b == 16 * (131072 * 4 * 128 * 2 + (128 * 128 + 128) * 4)
    assert abs(roofline.hbm_time_s(b) * 1e6 - 268.6) < 0.5


def test_decode_bytes():
    w = synth.WORKLOADS["decode_b256h32_d128"]
    per_head = roofline.decode_bytes(1, 1, w.Dk, w.Dv, 2)
    assert per_head == 2 * (128 * 128 + 128) * 4 + 4 * 128 * 2 == 133120


def test_streams_are_per_head_and_reproducible():
    a = synth.normal_heads(7, synth.Q_ID, 2, 3, 5, 4, 0.5, torch.float32)
    b = synth.normal_heads(7, synth.Q_ID, 2, 3, 5, 4, 0.5, torch.float32, heads=[(1, 2), (0, 1)])
    assert torch.equal(a[1, 2], b[0]) and torch.equal(a[0, 1], b[1])
    c = synth.normal_heads(7, synth.K_ID, 2, 3, 5, 4, 0.5, torch.float32)
    assert not torch.equal(a, c)
    # scaling happens in fp32 before rounding, bf16 is round-to-nearest-even of that
    raw = synth.normal_heads(7, synth.Q_ID, 2, 3, 5, 4, 1.0, torch.float32)
    bf = synth.normal_heads(7, synth.Q_ID, 2, 3, 5, 4, 0.5, torch.bfloat16)
    assert torch.equal(bf, (raw * np.float32(0.5)).to(torch.bfloat16))


def test_gate_recipe():
    a = synth.gate_heads(5, 1, 2, 4000)
    assert a.dtype == torch.float32 and a.shape == (1, 2, 4000)
    assert float(a.min()) > 0.0 and float(a.max()) < 1.0
    # g ~ N(4, 1): mean of -log(alpha) = E[log(1 + e^-g)] ~ 0.03
    m = float((-torch.log(a.double())).mean())
    assert 0.02 < m < 0.04


def test_workload_table():
    w = synth.WORKLOADS
    assert (w["tiny_fp32"].N, w["tiny_fp32"].Dk, w["tiny_fp32"].dtype) == (64, 16, torch.float32)
    assert w["b4h8_n4096_d64"].v_scale == 1.0 and w["b4h8_n4096_d64"].q_scale == 0.125
    assert w["long_n131072_d128"].v_scale == pytest.approx(1 / math.sqrt(128))
    assert w["decode_b256h32_d128"].prefix == 2048
    assert w["gated_b2h16_n16384_d128"].gated
