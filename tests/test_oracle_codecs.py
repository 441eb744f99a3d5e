"""Pins of the oracle's bf16 and E4M3FN codecs.

Fixed points of the OCP E4M3 definition (hand-listed values), a library
cross-check against torch.float8_e4m3fn (an independent implementation) on
every code and on in-range quantization, exhaustive round trips, ties and
saturation."""

import math

import numpy as np
import torch

from oracle import codecs

# (code, value) from the field definitions: bias 7, 3 mantissa bits, no inf
KNOWN = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x46, 3.5), (0x4C, 6.0),
    (0x70, 128.0), (0x77, 240.0), (0x78, 256.0), (0x7E, 448.0),
    (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
]


def test_known_codes():
    for code, val in KNOWN:
        assert codecs.e4m3_decode_scalar(code) == val, hex(code)
    assert math.isnan(codecs.e4m3_decode_scalar(0x7F))
    assert math.isnan(codecs.e4m3_decode_scalar(0xFF))
    neg_zero = codecs.e4m3_decode_scalar(0x80)
    assert neg_zero == 0.0 and math.copysign(1.0, neg_zero) < 0


def test_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2


def test_round_trip_every_finite_code():
    for c in range(256):
        v = codecs.e4m3_decode_scalar(c)
        if math.isnan(v):
            assert codecs.e4m3_encode_f64(v) & 0x7F == 0x7F
            continue
        assert codecs.e4m3_encode_f64(v) == c, hex(c)


def test_ties_go_to_even_mantissa():
    # midpoint between 1.0 (0x38, mantissa 0) and 1.125 (0x39, mantissa 1)
    assert codecs.e4m3_encode_f64(1.0625) == 0x38
    # midpoint between 1.125 (0x39) and 1.25 (0x3A, even) -> 0x3A
    assert codecs.e4m3_encode_f64(1.1875) == 0x3A
    # subnormal midpoint between 1 and 2 units of 2**-9 -> 2 (even)
    assert codecs.e4m3_encode_f64(1.5 * 2.0 ** -9) == 0x02
    # below half of the smallest subnormal -> zero, sign kept
    assert codecs.e4m3_encode_f64(0.49 * 2.0 ** -9) == 0x00
    assert codecs.e4m3_encode_f64(-0.49 * 2.0 ** -9) == 0x80
    # exact half of the smallest subnormal ties to zero (even)
    assert codecs.e4m3_encode_f64(0.5 * 2.0 ** -9) == 0x00
    # rounding that carries into the next binade: 1.9375 -> 2.0
    assert codecs.e4m3_encode_f64(1.96875) == 0x40


def test_saturation():
    assert codecs.e4m3_encode_f64(448.0) == 0x7E
    assert codecs.e4m3_encode_f64(449.0) == 0x7E
    assert codecs.e4m3_encode_f64(1e30) == 0x7E
    assert codecs.e4m3_encode_f64(-1e30) == 0xFE
    assert codecs.e4m3_encode_f64(math.inf) == 0x7E
    assert codecs.e4m3_encode_f64(-math.inf) == 0xFE
    assert codecs.e4m3_encode_f64(math.nan) == 0x7F


def test_quantize_matches_torch_in_range_exhaustive_bf16():
    # every bf16 bit pattern, several scales; compare where torch does not
    # overflow (|x / s| < 464: torch returns NaN above, the oracle saturates)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = codecs.bf16_bits_to_f64(bits).astype(np.float32)
    finite = np.isfinite(x)
    for s in (1.0, 2.0 ** -3, 0.37, 3.1):
        s32 = np.float32(s)
        quot = (x / s32).astype(np.float32)
        ok = finite & (np.abs(quot) < 464.0)
        ours = codecs.e4m3_quantize(x[ok], s32)
        ref = torch.from_numpy(quot[ok]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, ref), s
        # and the saturating region is all max-magnitude codes
        big = finite & (np.abs(quot) >= 464.0)
        sat = codecs.e4m3_quantize(x[big], s32)
        assert np.all((sat & 0x7F) == 0x7E)


def test_bf16_decode_is_exact():
    vals = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0], dtype=np.float32)
    bits = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(codecs.bf16_bits_to_f64(bits), ref)
