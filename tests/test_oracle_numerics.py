"""Pins for the oracle's number formats and its fp32 exp / SiLU specification.

bf16 rounding and the e4m3 codec are checked against torch's own conversions
(a library routine the oracle does not call) over every bf16 bit pattern;
exp32 and silu32 are checked against float64 math.
"""
import math

import numpy as np
import torch

from oracle import numerics as nm

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _finite_bf16_values():
    f = nm.bf16_to_f32(ALL_BF16)
    return f[np.isfinite(f)]


def test_bf16_decode_closed_form():
    for bits, val in [(0x3F80, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -133), (0x7F7F, 3.3895313892515355e38),
                      (0x3F81, 1.0 + 2 ** -7), (0x8000, -0.0)]:
        assert nm.bf16_to_f32(np.array([bits], np.uint16))[0] == np.float32(val)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * 10.0, rng.standard_normal(50000) * 1e-39,
                        rng.standard_normal(50000) * 1e30, [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nm.to_bf16(x32), ref)
    # float64 inputs are rounded once: a value just above a bf16 midpoint must round up
    # even when the float32 nearest to it is the midpoint itself
    mid = 1.0 + 2 ** -8
    assert nm.to_bf16(np.array([mid + 2 ** -40]))[0] == 0x3F81
    assert nm.to_bf16(np.array([mid]))[0] == 0x3F80            # tie -> even


def test_e4m3_encode_matches_torch_on_every_bf16():
    f = _finite_bf16_values()
    v = f[np.abs(f) <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(nm.e4m3_encode(v), ref)


def test_e4m3_encode_random_fp32_matches_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 300000), rng.standard_normal(300000) * 0.02,
                        rng.standard_normal(100000) * 2 ** -8]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(nm.e4m3_encode(v), ref)


def test_e4m3_decode_closed_form_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    dec = nm.e4m3_decode(codes)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if (c & 0x7F) == 0x7F:
            assert math.isnan(dec[c])
            continue
        ref = s * (m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
        assert dec[c] == ref
    assert dec[0x7E] == 448.0 and dec[0x38] == 1.0 and dec[0x01] == 2.0 ** -9
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    fin = ~np.isnan(dec)
    assert np.array_equal(dec[fin], ref[fin].astype(np.float64))
    # every finite code encodes back to itself (sign of zero kept)
    assert np.array_equal(nm.e4m3_encode(dec[fin]), codes[fin])


def test_e4m3_saturates_and_ties():
    assert nm.e4m3_encode(np.array([464.0, 470.0, 1e6, -1e6]))[:].tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    # halfway between 1.0 (0x38) and 1.125 (0x39) -> even mantissa 0x38; 1.1875 -> 0x3A
    assert nm.e4m3_encode(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10])).tolist() == \
        [0x38, 0x3A, 0x00, 0x02]


def test_exp32_within_one_ulp_over_all_bf16_inputs():
    x = _finite_bf16_values()
    x = x[(x >= -86.0) & (x <= 88.0)]
    got = nm.exp32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) <= 1.0


def test_exp32_clamps_and_special_points():
    assert nm.exp32(np.array([0.0], np.float32))[0] == np.float32(1.0)
    big = nm.exp32(np.array([1000.0, 88.0], np.float32))
    assert big[0] == big[1] and np.isfinite(big[0])
    small = nm.exp32(np.array([-1000.0, -86.0], np.float32))
    assert small[0] == small[1] and small[0] > 0


def test_silu32_against_float64():
    x = _finite_bf16_values()
    x = x[np.abs(x) <= 80.0]
    got = nm.silu32(x).astype(np.float64)
    x64 = x.astype(np.float64)
    ref = x64 / (1.0 + np.exp(-x64))
    tiny = np.abs(ref) < 1e-30
    ulp = np.spacing(np.abs(ref[~tiny]).astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got[~tiny] - ref[~tiny]) / ulp) <= 3.0
    # silu(0) = 0, silu(g) = g once exp(-g) < 2^-25, and silu(-g) = silu(g) - g
    assert nm.silu32(np.array([0.0], np.float32))[0] == 0.0
    assert nm.silu32(np.array([20.0, 64.0], np.float32)).tolist() == [20.0, 64.0]
    g = np.linspace(-6, 6, 1001).astype(np.float32)
    np.testing.assert_allclose(nm.silu32(-g), nm.silu32(g) - g, atol=2e-6)


def test_silu_closed_forms_outside_the_middle_range():
    """The SiLU specification reduces to closed forms outside |g| in [2^-25, 128):
    exp(-g) rounds to exactly 1 below (silu = g/2), 1 + exp(-g) rounds to 1 for
    g >= 128 (silu = g), and for g <= -128 the exponent argument saturates at 88,
    so silu(g) = g / D for one constant D and scales exactly with powers of two
    of g. Checked over every finite bf16 value (kernels that tabulate only the
    middle range rely on these)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    e = (bits.astype(np.uint32) >> 7) & 0xFF
    finite = e != 0xFF
    g = nm.bf16_to_f32(bits)
    s = nm.silu32(g)
    tiny = finite & (e < 102)
    assert np.array_equal(s[tiny].view(np.uint32), (g[tiny] * np.float32(0.5)).view(np.uint32))
    pos_big = finite & (e >= 134) & (bits < 0x8000)
    assert np.array_equal(s[pos_big].view(np.uint32), g[pos_big].view(np.uint32))
    neg_big = finite & (e >= 134) & (bits >= 0x8000)
    base = (bits[neg_big].astype(np.uint32) & 0x807F) | (134 << 7)        # same sign and mantissa, exponent of [128, 256)
    s_base = nm.silu32(nm.bf16_to_f32(base.astype(np.uint16)))
    scaled = np.ldexp(s_base, (e[neg_big].astype(np.int32) - 134)).astype(np.float32)
    assert np.array_equal(s[neg_big].view(np.uint32), scaled.view(np.uint32))
    # and the middle range is exactly what a table of 2 * 32 * 128 entries must hold
    mid = finite & (e >= 102) & (e < 134)
    assert mid.sum() == 2 * 32 * 128
