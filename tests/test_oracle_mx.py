"""Pins of the MXFP8 reference (oracle/mx.py) against facts that do not come
from the reference itself: the E4M3 format's defining values, an independent
library conversion (torch's float8_e4m3fn cast) for every in-range value
class, the scale rule on crafted blocks, brute-force nearest search, and the
rounding error bound."""
import numpy as np
import pytest
import torch

from oracle import mx

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_e4m3_defining_values():
    # format facts: bias 7, 3 mantissa bits, max finite 448, min normal 2^-6,
    # min subnormal 2^-9, NaN only at S.1111.111, sign-magnitude
    assert mx.e4m3_value(0x00) == 0.0
    assert mx.e4m3_value(0x38) == 1.0
    assert mx.e4m3_value(0x7E) == 448.0
    assert mx.e4m3_value(0x08) == 2.0 ** -6
    assert mx.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert mx.e4m3_value(0x01) == 2.0 ** -9
    assert mx.e4m3_value(0x78) == 256.0
    assert mx.e4m3_value(0xB8) == -1.0
    assert np.isnan(mx.e4m3_value(0x7F)) and np.isnan(mx.e4m3_value(0xFF))
    vals = mx.e4m3_value(np.arange(256))
    assert np.sum(np.isnan(vals)) == 2
    # 126 distinct positive finite values plus zero, mirrored by the sign
    assert len(np.unique(vals[:0x7F])) == 127
    np.testing.assert_array_equal(vals[0x80:0xFF], -vals[:0x7F])


def test_decode_matches_torch_float8_bit_reinterpretation():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = mx.e4m3_value(np.arange(256))
    same = (lib == ours) | (np.isnan(lib) & np.isnan(ours))
    assert same.all()


def test_encode_matches_torch_cast_in_range():
    # every representable value, every midpoint between neighbours (ties),
    # points near the midpoints, and random values; all below 464 where the
    # library cast (which does not saturate) and ours agree by definition
    pos = mx.e4m3_value(np.arange(0x7F))
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(0)
    rnd = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(460.0), 20000))
    x = np.concatenate([pos, mids, mids * (1 + 1e-9), mids * (1 - 1e-9), rnd, [455.0, 463.9]])
    x = np.concatenate([x, -x])
    lib = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # the float32 cast of the float64 input is exact for all but the +-1e-9
    # nudges, whose float32 value stays on the same side of the midpoint
    ours = mx.e4m3_encode(x.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(ours, lib)


def test_encode_ties_saturation_and_signed_zero():
    assert mx.e4m3_encode(1.0625) == 0x38        # tie 1.0 / 1.125 -> even 1.0
    assert mx.e4m3_encode(1.1875) == 0x3A        # tie 1.125 / 1.25 -> even 1.25
    assert mx.e4m3_encode(17.0) == 0x58          # tie 16 / 18 -> 16
    assert mx.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie 2^-9 / 2^-8 -> 2^-8
    assert mx.e4m3_encode(2.0 ** -10) == 0x00    # tie 0 / 2^-9 -> 0
    assert mx.e4m3_encode(7.5 * 2.0 ** -9) == 0x08  # subnormal/normal tie -> 2^-6
    for big in (448.0, 450.0, 464.0, 500.0, 511.99, 1e30, np.inf):
        assert mx.e4m3_encode(big) == 0x7E and mx.e4m3_encode(-big) == 0xFE
    assert mx.e4m3_encode(-0.0) == 0x80 and mx.e4m3_encode(-1e-30) == 0x80


def test_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(3000) * rng.choice([1e-3, 0.1, 10, 300], 3000)
    codes = mx.e4m3_encode(x)
    allv = mx.e4m3_value(np.arange(256))
    fin = ~np.isnan(allv)
    for xi, ci in zip(x, codes):
        d = np.abs(allv[fin] - np.clip(xi, -448, 448))
        assert abs(mx.e4m3_value(ci) - np.clip(xi, -448, 448)) == d.min()


def test_shared_exponent_rule():
    # the block maximum lands in [256, 512) after scaling
    assert mx.shared_exponent(1.0) == -8
    assert mx.shared_exponent(1.75) == -8        # 1.75 * 2^8 = 448 exactly
    assert mx.shared_exponent(1.99) == -8        # 509.4: saturates to 448
    assert mx.shared_exponent(2.0) == -7
    assert mx.shared_exponent(0.03) == -14       # floor(log2 0.03) = -6
    assert mx.shared_exponent(0.0) == -126
    assert mx.shared_exponent(2.0 ** -120) == -126
    rng = np.random.default_rng(2)
    amax = np.exp(rng.uniform(-20, 20, 1000))
    se = mx.shared_exponent(amax)
    scaled = amax * np.exp2(-se.astype(float))
    assert np.all((scaled >= 256) & (scaled < 512))


def test_block_quantize_crafted():
    w = np.zeros((2, 64))
    w[0, :32] = np.linspace(-1.0, 1.0, 32)       # max 1.0 -> scale 2^-8
    w[0, 32:] = 0.0                              # all-zero block
    w[1, :32] = 1.75                             # exactly 448 after scaling
    w[1, 32:] = 3 * 2.0 ** -18                   # 1.5 * 2^-17: shared exponent -25
    codes, scales = mx.quantize(w)
    assert scales.tolist() == [[119, 1], [119, 102]]
    assert codes[0, 31] == 0x78 and codes[0, 0] == 0xF8       # +-256
    assert (codes[0, 32:] == 0).all()
    assert (codes[1, :32] == 0x7E).all()
    assert (codes[1, 32:] == 0x7C).all()          # 1.5 * 2^8 = 384: E=15, m=4
    np.testing.assert_array_equal(mx.dequantize(codes, scales)[1, :32], 1.75)


def test_roundtrip_error_bound_and_exact_values():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((64, 256)) / 48
    codes, scales = mx.quantize(w)
    dq = mx.dequantize(codes, scales)
    X = np.repeat(np.exp2(scales.astype(float) - 127), 32, axis=1)
    a = np.abs(w) / X                             # scaled magnitudes
    # normal range: half an ulp of a 3-bit mantissa (2^-4 relative);
    # subnormal range: half of 2^-9 (absolute, in scaled units)
    err = np.abs(dq - w) / X
    sat = a > 448
    normal = (a >= 2.0 ** -6) & ~sat
    assert np.all(err[normal] <= a[normal] * 2.0 ** -4 * (1 + 1e-12))
    assert np.all(err[a < 2.0 ** -6] <= 2.0 ** -10 * (1 + 1e-12))
    # saturated block maxima (scaled into (448, 512)) clip to 448
    np.testing.assert_allclose(err[sat], a[sat] - 448, rtol=1e-12)
    assert sat.any()
    # values that are already E4M3 x 2^e come back unchanged
    exact = mx.dequantize(codes, scales)
    c2, s2 = mx.quantize(exact)
    np.testing.assert_array_equal(mx.dequantize(c2, s2), exact)


def test_dequantized_values_are_bf16_exact():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((8, 128)) / 30
    dq = mx.dequantize(*mx.quantize(w)).astype(np.float32)
    as_bf16 = torch.from_numpy(dq).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(as_bf16, dq)


def test_quantized_weight_fn_touches_only_matrices():
    calls = []

    def weight(name):
        calls.append(name)
        return np.full((4, 32), 0.3) if name.endswith(("w_o", "alpha")) else np.ones(32)
    f = mx.quantized_weight_fn(weight)
    assert not np.array_equal(f("sub0.w_o"), np.full((4, 32), 0.3))   # 0.3 is not E4M3 x 2^e
    np.testing.assert_array_equal(f("sub0.alpha"), np.full((4, 32), 0.3))
    np.testing.assert_array_equal(f("embed"), np.ones(32))
