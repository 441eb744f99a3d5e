"""Stored-scalar codecs: bf16 and OCP E4M3FN, in float64.

Page 2, "KV Cache Explained", section "What changes when you use FP8 KV":
FP8 stores one byte per element and quantized values need scales.  The pages
fix neither the bit format nor the rounding, so this module follows the OCP
8-bit floating point specification's E4M3 encoding (called E4M3FN in most
libraries):

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 encodes subnormals m * 2**-9;
* no infinities; S.1111.111 is NaN; the largest finite magnitude is
  1.75 * 2**8 = 448.

Quantization of a stored value x with scale s is RNE_sat(fp32(x) / fp32(s)):
the quotient is formed in IEEE float32 (correctly rounded), then rounded to
the nearest E4M3 value with ties to an even mantissa, saturating at +-448.
A NaN quotient maps to the NaN code with the input's sign.

bf16 is the upper half of an IEEE float32: decoding shifts the 16 stored bits
left by 16.
"""

from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# E4M3FN
# --------------------------------------------------------------------------

def e4m3_decode_scalar(code: int) -> float:
    """Value of one E4M3FN code, from the field definitions."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man = code & 0x7
    if exp_field == 0xF and man == 0x7:
        return math.nan
    if exp_field == 0:
        return sign * man * 2.0 ** -9          # subnormal: 0.mmm * 2**(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp_field - 7)


_E4M3_TABLE = np.array([e4m3_decode_scalar(c) for c in range(256)],
                       dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN codes (uint8 array) -> float64 values (exact)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def _round_half_even(v: float) -> float:
    f = math.floor(v)
    d = v - f
    if d > 0.5:
        return f + 1.0
    if d < 0.5:
        return f
    return f if (f % 2 == 0) else f + 1.0


def e4m3_encode_f64(v: float) -> int:
    """Nearest E4M3FN code to the real value ``v`` (ties to even mantissa,
    saturating to +-448, NaN to the NaN code)."""
    if math.isnan(v):
        return E4M3_NAN | (0x80 if math.copysign(1.0, v) < 0 else 0)
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a >= E4M3_MAX:
        return sign | 0x7E                      # 448 = 1.110b * 2**8
    # Quantum: 2**-9 in the subnormal range and the lowest binade (|a| < 2**-5
    # covers both since 2**-6 .. 2**-5 also has quantum 2**-9); 2**(e-3) above.
    if a < 2.0 ** -6:
        quantum = 2.0 ** -9
    else:
        e = math.floor(math.log2(a))
        # guard against log2 rounding at exact powers of two
        if 2.0 ** e > a:
            e -= 1
        elif 2.0 ** (e + 1) <= a:
            e += 1
        quantum = 2.0 ** (e - 3)
    r = _round_half_even(a / quantum) * quantum
    if r > E4M3_MAX:                            # cannot happen below 448, kept for clarity
        r = E4M3_MAX
    if r == 0.0:
        return sign
    # find the code of r by its fields
    if r < 2.0 ** -6:
        return sign | int(round(r / 2.0 ** -9))
    e = math.floor(math.log2(r))
    if 2.0 ** e > r:
        e -= 1
    man = int(round((r / 2.0 ** e - 1.0) * 8.0))
    if man == 8:                                # rounding carried into the exponent
        man = 0
        e += 1
    return sign | ((e + 7) << 3) | man


def e4m3_quantize(x_f32, scale_f32) -> np.ndarray:
    """RNE_sat(fp32(x) / fp32(scale)) -> uint8 codes, elementwise.

    The division is done in IEEE float32 (numpy float32 arithmetic is
    correctly rounded), then each quotient is rounded to E4M3FN exactly."""
    x = np.asarray(x_f32, dtype=np.float32)
    s = np.asarray(scale_f32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        q = (x / s).astype(np.float32)
    flat = q.astype(np.float64).ravel()
    out = np.fromiter((e4m3_encode_f64(float(v)) for v in flat),
                      dtype=np.uint8, count=flat.size)
    return out.reshape(q.shape)
