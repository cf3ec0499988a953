"""Pins of the oracle's low-precision state (the decode step with S, z stored in bf16 or fp8).

- The rounding to a storage type is checked against the library conversions
  (torch bfloat16 and float8_e4m3fn, round to nearest even; float8_e4m3fn has
  no infinity and turns magnitudes past 448 into NaN, as the gfx950
  conversion does) on values across the whole range, subnormals included.
- With an fp32 state the step is the plain decode step up to fp32 rounding.
- When every value stays exactly representable the stored recurrence is the
  exact one, bit for bit.
- Round to nearest even stalls a bf16 sum of ones at 256 (256 + 1 is a tie
  between 256 and 258): the running normalizer of an ungated summary stops
  growing, which is the accumulation the product-order page warns about.
"""
import numpy as np
import pytest
import torch

import oracle


def grid():
    r = np.random.default_rng(41)
    mags = np.ldexp(r.uniform(1.0, 2.0, 6000), r.integers(-20, 12, 6000))
    x = np.concatenate([mags, -mags, [0.0, 448.0, 464.0, 480.0, 1000.0, 2.0 ** -9, 3 * 2.0 ** -10, 1.0625]])
    return x.astype(np.float32).astype(np.float64)  # values the library rounds are fp32


@pytest.mark.parametrize("dtype,code", [(torch.bfloat16, oracle.STATE_BF16), (torch.float8_e4m3fn, oracle.STATE_FP8_E4M3)])
def test_state_rounding_matches_the_library_conversion(dtype, code):
    x = grid()
    ref = torch.from_numpy(x.astype(np.float32)).to(dtype).double().numpy()
    got = oracle.state_round(x, code)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), x[~same][:10]


def inputs(B, H, Dk, Dv, seed, scale=0.1):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, H, Dk)) * scale, r.standard_normal((B, H, Dk)) * scale,
            r.standard_normal((B, H, Dv)))


def test_fp32_state_is_the_plain_step():
    s = np.zeros((2, 3, 16, 8))
    z = np.zeros((2, 3, 16))
    s2, z2 = s.copy(), z.copy()
    for t in range(20):
        q, k, v = inputs(2, 3, 16, 8, seed=100 + t)
        o, s, z = oracle.decode_step(q, k, v, s, z)
        o2, s2, z2 = oracle.decode_lowp(q, k, v, s2, z2, oracle.STATE_F32)
        np.testing.assert_allclose(s2, s, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(o2, o, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("code", [oracle.STATE_BF16, oracle.STATE_FP8_E4M3])
def test_exactly_representable_recurrence_is_exact(code):
    # identity map, 0/1 keys and queries, values in {-1, 0, 1}: every state
    # entry is a small integer (at most 12 in magnitude, exact in fp8 too)
    r = np.random.default_rng(42)
    s = np.zeros((1, 2, 8, 4))
    z = np.zeros((1, 2, 8))
    s_ref, z_ref = s.copy(), z.copy()
    for t in range(12):
        q = r.integers(0, 2, (1, 2, 8)).astype(float)
        k = r.integers(0, 2, (1, 2, 8)).astype(float)
        v = r.integers(-1, 2, (1, 2, 4)).astype(float)
        o, s, z = oracle.decode_lowp(q, k, v, s, z, code, phi_mode=oracle.PHI_IDENTITY)
        o_ref, s_ref, z_ref = oracle.decode_step(q, k, v, s_ref, z_ref, phi_mode=oracle.PHI_IDENTITY)
        np.testing.assert_array_equal(s, s_ref)
        np.testing.assert_array_equal(z, z_ref)
        np.testing.assert_allclose(o, o_ref, rtol=1e-15)


def test_bf16_sum_of_ones_stalls_at_256():
    s = np.zeros((1, 1, 1, 1))
    z = np.zeros((1, 1, 1))
    one = np.ones((1, 1, 1))
    for t in range(300):
        _, s, z = oracle.decode_lowp(one, one, one, s, z, oracle.STATE_BF16, phi_mode=oracle.PHI_IDENTITY)
    assert z[0, 0, 0] == 256.0 and s[0, 0, 0, 0] == 256.0
