"""Number encodings of the packed weight formats (oracle; test infrastructure only).

The subject pages name the encodings but do not define them: the NInfer
article (section 2) and the Decapybara kernel list speak of NVFP4 weights
(FP4 E2M1 values with an FP8 E4M3 scale), the NInfer article (section 4)
names FP8 E4M3, and the groupwise-int formats carry fp16 scale fields. The
definitions used here are the public ones:

  * IEEE 754 binary16 (fp16): 1 sign, 5 exponent (bias 15), 10 mantissa bits.
  * bfloat16: the upper half of an IEEE binary32.
  * OCP FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits, subnormals,
    no infinities, only S.1111.111 is NaN, largest finite 448.
  * OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit, magnitudes
    {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code 8 is negative zero.
  * OCP E8M0 (the shared scale of the OCP microscaling (MX) formats, which the
    Decapybara kernel list names for its MXFP8 GEMV and activation
    quantiser): 8 exponent bits, bias 127, no sign and no mantissa, value
    2^(bits - 127); 0xFF is NaN.

Two independent implementations live here:
  * exact_* functions work on fractions.Fraction and round by the textbook
    rule (nearest, ties to the even significand), for tiny inputs and pins;
  * the numpy functions are vectorised and serve large inputs. Tests check
    the second against the first.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# ---------------------------------------------------------------------------
# Exact rounding to a binary floating-point format
# ---------------------------------------------------------------------------


def _floor_log2(a: Fraction) -> int:
    """Largest e with 2**e <= a, for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def exact_round(v, p: int, emin: int, maxfinite: Fraction, saturate: bool):
    """Round the rational v to a binary format, nearest with ties to even.

    p         significand bits including the hidden bit
    emin      exponent of the smallest normal number (subnormals below it)
    maxfinite largest finite magnitude
    saturate  clamp out-of-range magnitudes to maxfinite instead of infinity

    Returns a Fraction, or +-math.inf on (non-saturating) overflow. The sign
    of a zero result is not represented; callers carry the sign separately.
    """
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - (p - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r > maxfinite:
        if saturate:
            r = maxfinite
        else:
            return sign * math.inf
    return sign * r


F16_MAX = Fraction(65504)
BF16_MAX = Fraction(2 ** 8 - 1, 2 ** 7) * Fraction(2) ** 127
F32_MAX = Fraction(2 ** 24 - 1, 2 ** 23) * Fraction(2) ** 127
F64_MAX = Fraction(2 ** 53 - 1, 2 ** 52) * Fraction(2) ** 1023
E4M3_MAX = Fraction(448)
E2M1_MAX = Fraction(6)


def exact_round_f16(v):
    return exact_round(v, 11, -14, F16_MAX, False)


def exact_round_f32(v):
    return exact_round(v, 24, -126, F32_MAX, False)


def exact_round_f64(v):
    return exact_round(v, 53, -1022, F64_MAX, False)


def exact_round_e4m3_sat(v):
    return exact_round(v, 4, -6, E4M3_MAX, True)


def exact_round_e2m1_sat(v):
    return exact_round(v, 2, 0, E2M1_MAX, True)


# ---------------------------------------------------------------------------
# Exact decoders (bit pattern -> value) written from the field definitions
# ---------------------------------------------------------------------------


def exact_f16_value(bits: int):
    """fp16 bit pattern -> Fraction (or float inf / nan)."""
    s, e, m = (bits >> 15) & 1, (bits >> 10) & 0x1F, bits & 0x3FF
    if e == 0x1F:
        return math.nan if m else (-math.inf if s else math.inf)
    mag = Fraction(m, 2 ** 24) if e == 0 else Fraction(1024 + m) * Fraction(2) ** (e - 25)
    return -mag if s else mag


def exact_bf16_value(bits: int):
    s, e, m = (bits >> 15) & 1, (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0xFF:
        return math.nan if m else (-math.inf if s else math.inf)
    mag = Fraction(m) * Fraction(2) ** -133 if e == 0 else Fraction(128 + m) * Fraction(2) ** (e - 134)
    return -mag if s else mag


def exact_e4m3_value(bits: int):
    s, e, m = (bits >> 7) & 1, (bits >> 3) & 0xF, bits & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    mag = Fraction(m, 512) if e == 0 else Fraction(8 + m) * Fraction(2) ** (e - 10)
    return -mag if s else mag


def exact_e8m0_value(bits: int):
    """E8M0 byte -> Fraction 2^(bits - 127), or float nan for 0xFF."""
    if not 0 <= bits <= 0xFF:
        raise ValueError("E8M0 is one byte")
    if bits == 0xFF:
        return math.nan
    return Fraction(2) ** (bits - 127)


def exact_e2m1_value(bits: int):
    s, e, m = (bits >> 3) & 1, (bits >> 1) & 0x3, bits & 0x1
    mag = Fraction(m, 2) if e == 0 else Fraction(2 + m) * Fraction(2) ** (e - 2)
    return -mag if s else mag


# ---------------------------------------------------------------------------
# Exact encoders (value -> bit pattern); the value must already be representable
# ---------------------------------------------------------------------------


def _exact_bits(mag: Fraction, p: int, emin: int, bias: int, ebits: int) -> int:
    """Exponent/mantissa fields of a representable positive magnitude."""
    mbits = p - 1
    if mag == 0:
        return 0
    e = _floor_log2(mag)
    if e < emin:  # subnormal
        m = mag / Fraction(2) ** (emin - mbits)
        assert m.denominator == 1 and 0 < m < 2 ** mbits
        return int(m)
    m = mag / Fraction(2) ** (e - mbits) - 2 ** mbits
    assert m.denominator == 1 and 0 <= m < 2 ** mbits
    ef = e + bias
    assert 0 < ef < 2 ** ebits
    return (ef << mbits) | int(m)


def exact_f16_bits(value, negative: bool = False) -> int:
    """Bits of an fp16-representable value (Fraction or +-inf)."""
    if isinstance(value, float) and math.isinf(value):
        return 0xFC00 if value < 0 else 0x7C00
    value = Fraction(value)
    s = 1 if (value < 0 or (value == 0 and negative)) else 0
    return (s << 15) | _exact_bits(abs(value), 11, -14, 15, 5)


def exact_e4m3_bits(value) -> int:
    value = Fraction(value)
    s = 1 if value < 0 else 0
    return (s << 7) | _exact_bits(abs(value), 4, -6, 7, 4)


def exact_e2m1_bits(value, negative: bool = False) -> int:
    value = Fraction(value)
    s = 1 if (value < 0 or (value == 0 and negative)) else 0
    return (s << 3) | _exact_bits(abs(value), 2, 0, 1, 2)


# ---------------------------------------------------------------------------
# Decode tables (closed forms above, evaluated once)
# ---------------------------------------------------------------------------


def _f(v, negative: bool) -> float:
    """Fraction (or float nan/inf) -> float, keeping the sign of a zero."""
    f = float(v) if not isinstance(v, float) else v
    return math.copysign(0.0, -1.0) if (f == 0 and negative) else f


E4M3_TABLE = np.array([_f(exact_e4m3_value(b), bool(b & 0x80)) for b in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_f(exact_e2m1_value(b), bool(b & 0x8)) for b in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([_f(exact_e8m0_value(b), False) for b in range(256)], dtype=np.float64)
# positive finite magnitudes in code order (codes 0..126 / 0..7 are increasing)
_E4M3_POS = E4M3_TABLE[:127].copy()
_E2M1_POS = E2M1_TABLE[:8].copy()


# ---------------------------------------------------------------------------
# Vectorised codecs (numpy)
# ---------------------------------------------------------------------------


def f16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bit patterns, one round-to-nearest-even (numpy's cast;
    magnitudes that round past 65504 become infinity)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_from_f16_bits(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def f64_from_f16_bits(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _nearest_even_code(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table value nearest to mag (ties -> even index).

    table: increasing non-negative magnitudes, index == code (the lowest code
    bit is the mantissa's lowest bit, so "even index" == "even significand").
    Magnitudes above the last entry saturate to it.
    """
    mag = np.asarray(mag, dtype=np.float64)
    lo = np.searchsorted(table, mag, side="right") - 1
    lo = np.clip(lo, 0, len(table) - 1)
    hi = np.minimum(lo + 1, len(table) - 1)
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    return np.where(mag >= table[-1], len(table) - 1, code).astype(np.uint8)


def e4m3_encode_sat(v: np.ndarray) -> np.ndarray:
    """Non-negative values -> OCP E4M3 codes, nearest-even, saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("E4M3 scale inputs must be non-negative numbers")
    return _nearest_even_code(v, _E4M3_POS)


def e2m1_encode_sat(v: np.ndarray) -> np.ndarray:
    """Values -> OCP E2M1 codes, nearest-even, saturating at +-6.

    The sign bit follows the sign bit of the input, so a negative input that
    rounds to zero gives code 8 (negative zero), as an IEEE rounding would.
    """
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_even_code(np.abs(v), _E2M1_POS)
    return (mag | (np.signbit(v).astype(np.uint8) << np.uint8(3))).astype(np.uint8)


def e4m3_encode_signed_sat(v: np.ndarray) -> np.ndarray:
    """Values -> OCP E4M3 codes, nearest-even, saturating at +-448; the sign
    bit follows the input's sign bit (a negative input that rounds to zero,
    and -0, give code 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("E4M3 element inputs must be numbers")
    mag = _nearest_even_code(np.abs(v), _E4M3_POS)
    return (mag | (np.signbit(v).astype(np.uint8) << np.uint8(7))).astype(np.uint8)


def e8m0_decode(bits: np.ndarray) -> np.ndarray:
    """E8M0 bytes -> float64 2^(bits - 127) (nan for 0xFF); exact."""
    return E8M0_TABLE[np.asarray(bits, dtype=np.uint8)]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & np.uint8(0xF)]
