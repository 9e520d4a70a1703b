"""Per-format quantisers (oracle; test infrastructure only).

The pages fix which formats exist, not how they are produced:
  * NInfer article, section 2: the 27B groupwise-int recipe puts some
    projections in 4-bit and others in 5-bit groupwise integers, and the
    NVFP4 artefact imports 4-bit weights directly;
  * RustingStrata page, format list: a Q8_0-style symmetric 8-bit format;
  * Decapybara page, kernel list: NVFP4 GEMV (E2M1 values with E4M3 block
    scales).
Where the pages are silent, the plainest reading is taken (each one is
listed with the design notes of the repository):
  * asymmetric int (4/5 bit), 32 weights per group along K:
        w ~= d * q + m,  q in [0, 2^b - 1],  m = group minimum,
        d = fp16((max - min) / (2^b - 1)) with the subtraction and division
        done in fp32, m = fp16(min), q = clamp(rint((w - m) / d)) in fp64
        (ties to even), q = 0 when d == 0;
  * symmetric int8, 32 per group: d = fp16(amax / 127) in fp32,
        q = clamp(rint(w / d), -127, 127) in fp64, q = 0 when d == 0;
  * MXFP8 / MXFP4 (OCP microscaling; the Decapybara kernel list names an
        MXFP8 block-scaled GEMV and a dynamic 32-element MXFP8 activation
        quantiser): per 32 values along K one E8M0 scale 2^X with
        X = floor(log2(amax)) - emax, emax = 8 (E4M3: 448 = 1.75 * 2^8) or
        2 (E2M1: 6 = 1.5 * 2^2), clamped to [-127, 127], X = -127 when
        amax == 0; elements = E4M3 / E2M1 of w / 2^X (exact in fp64),
        nearest-even, saturating; the sign bit follows the input's;
  * NVFP4: tensor scale s_t = amax / (6 * 448) in fp32 (1 when that is 0),
        block scale (16 weights along K) b = E4M3(amax_b / (6 * s_t)) with the
        product and quotient in fp32, nearest-even, saturating;
        code = E2M1(w / (b * s_t)) in fp64, nearest-even, saturating; all
        codes of a block with b == 0 are +0.

Two implementations: `quantize` (numpy, whole matrices) and
`quantize_group_exact` (one group in exact rational arithmetic, emulating
each fp32 / fp64 operation by a correctly rounded step).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from . import encodings as enc

GROUP = 32          # weights per scale group along K (int formats)
MX_BLOCK = 32       # values per E8M0 scale along K (MX formats)
MX_EMAX = {"mxfp8": 8, "mxfp4": 2}   # exponent of the element format's top binade
NVFP4_BLOCK = 16    # weights per E4M3 block scale along K


class QuantRangeError(ValueError):
    """A scale field does not fit its encoding (fp16 overflow)."""


@dataclass
class Quantized:
    """Logical fields of a quantised [M][K] matrix (row m, column k).

    codes  uint8 [M][K] (int4: 0..15, int5: 0..31, nvfp4: E2M1 4-bit codes)
           or int8 [M][K] (int8 format)
    d      uint16 [M][K/32] fp16 bits of the scale (int formats)
    m      uint16 [M][K/32] fp16 bits of the minimum (asymmetric formats)
    sb     uint8  [M][K/16] E4M3 block scales (nvfp4)
    st     float32 tensor scale (nvfp4)
    e      uint8  [M][K/32] E8M0 block scales (mxfp8: codes are E4M3 bytes,
           mxfp4: codes are E2M1 4-bit codes)
    """
    fmt: str
    M: int
    K: int
    codes: np.ndarray
    d: np.ndarray | None = None
    m: np.ndarray | None = None
    sb: np.ndarray | None = None
    st: np.float32 | None = None
    e: np.ndarray | None = None


def _check(W: np.ndarray) -> tuple[int, int]:
    if W.dtype != np.float32 or W.ndim != 2:
        raise TypeError("W must be a float32 [M][K] array")
    M, K = W.shape
    if M < 1 or K < GROUP or K % GROUP:
        raise ValueError("need M >= 1 and K a positive multiple of 32")
    if not np.all(np.isfinite(W)):
        raise ValueError("weights must be finite")
    return M, K


def quantize(W: np.ndarray, fmt: str) -> Quantized:
    """Quantise a float32 [M][K] matrix. Negative zeros in W are first made
    +0 (an fp32 addition of +0), so that no field depends on which of two
    equal zeros a min/max reduction returns."""
    M, K = _check(W)
    W = W + np.float32(0.0)
    if fmt in ("int4", "int5"):
        bits = 4 if fmt == "int4" else 5
        qmax = (1 << bits) - 1
        Wg = W.reshape(M, K // GROUP, GROUP)
        mn = Wg.min(axis=2)
        mx = Wg.max(axis=2)
        with np.errstate(over="ignore"):
            d32 = (mx - mn) / np.float32(qmax)          # fp32 subtract, fp32 divide
            d16 = enc.f16_bits_from_f32(d32)
            m16 = enc.f16_bits_from_f32(mn)
        dd = enc.f64_from_f16_bits(d16)
        mm = enc.f64_from_f16_bits(m16)
        if not (np.all(np.isfinite(dd)) and np.all(np.isfinite(mm))):
            raise QuantRangeError("group scale or minimum overflows fp16")
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.rint((Wg.astype(np.float64) - mm[..., None]) / dd[..., None])
        q = np.where(dd[..., None] == 0.0, 0.0, q)
        q = np.clip(q, 0, qmax).astype(np.uint8).reshape(M, K)
        return Quantized(fmt, M, K, q, d=d16, m=m16)
    if fmt == "int8":
        Wg = W.reshape(M, K // GROUP, GROUP)
        amax = np.abs(Wg).max(axis=2)
        d32 = amax / np.float32(127.0)
        with np.errstate(over="ignore"):
            d16 = enc.f16_bits_from_f32(d32)
        dd = enc.f64_from_f16_bits(d16)
        if not np.all(np.isfinite(dd)):
            raise QuantRangeError("group scale overflows fp16")
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.rint(Wg.astype(np.float64) / dd[..., None])
        q = np.where(dd[..., None] == 0.0, 0.0, q)
        q = np.clip(q, -127, 127).astype(np.int8).reshape(M, K)
        return Quantized(fmt, M, K, q, d=d16)
    if fmt == "nvfp4":
        amax = np.abs(W).max()
        st = np.float32(amax / np.float32(2688.0))
        if st == 0:
            st = np.float32(1.0)
        Wb = W.reshape(M, K // NVFP4_BLOCK, NVFP4_BLOCK)
        amax_b = np.abs(Wb).max(axis=2)
        denom = np.float32(6.0) * st                      # fp32 product
        ratio = (amax_b / denom).astype(np.float32)       # fp32 quotient
        sb = enc.e4m3_encode_sat(ratio)
        sbv = enc.e4m3_decode(sb)                          # exact float64
        with np.errstate(divide="ignore", invalid="ignore"):
            v = Wb.astype(np.float64) / (sbv[..., None] * np.float64(st))
        codes = enc.e2m1_encode_sat(np.where(sbv[..., None] == 0.0, 0.0, v))
        codes = np.where(sbv[..., None] == 0.0, np.uint8(0), codes).astype(np.uint8)
        return Quantized(fmt, M, K, codes.reshape(M, K), sb=sb, st=st)
    if fmt in MX_EMAX:
        codes, e = mx_quantize_blocks(W.reshape(M, K // MX_BLOCK, MX_BLOCK), fmt)
        return Quantized(fmt, M, K, codes.reshape(M, K), e=e)
    raise ValueError(f"unknown format {fmt!r}")


def mx_scale_exponent(amax: np.ndarray, emax: int) -> np.ndarray:
    """X = floor(log2(amax)) - emax, clamped to [-127, 127]; -127 where
    amax == 0. frexp gives amax = f * 2^p with f in [0.5, 1), exactly, so
    floor(log2(amax)) = p - 1 for every positive finite amax."""
    amax = np.asarray(amax, dtype=np.float64)
    _, p = np.frexp(amax)
    X = np.where(amax == 0.0, -127, (p - 1) - emax)
    return np.clip(X, -127, 127).astype(np.int64)


def mx_quantize_blocks(V: np.ndarray, fmt: str) -> tuple[np.ndarray, np.ndarray]:
    """MX quantisation of blocks V[..., 32] (finite fp32 values): returns the
    element codes [..., 32] (uint8) and the E8M0 scale bytes [...]."""
    V = np.asarray(V)
    if V.shape[-1] != MX_BLOCK:
        raise ValueError("MX blocks hold 32 values")
    amax = np.abs(V.astype(np.float64)).max(axis=-1)
    X = mx_scale_exponent(amax, MX_EMAX[fmt])
    v = V.astype(np.float64) / np.ldexp(1.0, X)[..., None]      # exact: a power of two
    codes = enc.e4m3_encode_signed_sat(v) if fmt == "mxfp8" else enc.e2m1_encode_sat(v)
    return codes.astype(np.uint8), (X + 127).astype(np.uint8)


def mx_act_quant(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Dynamic MXFP8 quantisation of bf16 activations [N][K] (bit patterns;
    K a multiple of 32): E4M3 codes [N][K] and E8M0 scales [N][K/32], by the
    MXFP8 rule above. The sign of a zero input is kept (-0 -> code 0x80)."""
    x = enc.f32_from_bf16_bits(x_bits)
    N, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("activations must be finite")
    codes, e = mx_quantize_blocks(x.reshape(N, K // MX_BLOCK, MX_BLOCK), "mxfp8")
    return codes.reshape(N, K), e


def mx_block_exact(ws: list, fmt: str) -> tuple[list[int], int]:
    """One MX block in exact rational arithmetic: (element codes, E8M0 byte).
    A negative input (or -0.0) gives a negative-signed code."""
    vals = [Fraction(w) for w in ws]
    amax = max(abs(v) for v in vals)
    if amax == 0:
        X = -127
    else:
        X = max(-127, min(127, enc._floor_log2(amax) - MX_EMAX[fmt]))
    codes = []
    for w, v in zip(ws, vals):
        neg = v < 0 or (v == 0 and math.copysign(1.0, float(w)) < 0)
        if fmt == "mxfp8":
            c = enc.exact_e4m3_bits(enc.exact_round_e4m3_sat(abs(v) / Fraction(2) ** X)) | (0x80 if neg else 0)
        else:
            c = enc.exact_e2m1_bits(enc.exact_round_e2m1_sat(abs(v) / Fraction(2) ** X)) | (0x8 if neg else 0)
        codes.append(c)
    return codes, X + 127


# ---------------------------------------------------------------------------
# Exact single-group quantiser (pure Python, rationals)
# ---------------------------------------------------------------------------


def _rint_half_even(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def quantize_group_exact(ws: list[float], fmt: str, st: float | None = None):
    """Quantise one group exactly, emulating every fp32/fp64 step.

    ws: the group's weights as Python floats holding fp32 values (32 for the
    int formats, 16 for one NVFP4 block). For NVFP4 the tensor scale st
    (an fp32 value) is passed in. Returns (codes, fields) where fields is
    (d_bits, m_bits) / (d_bits,) / (sb_code,).
    """
    vals = [Fraction(w) for w in ws]
    if fmt in ("int4", "int5"):
        qmax = 15 if fmt == "int4" else 31
        mn, mx = min(vals), max(vals)
        d32 = enc.exact_round_f32(enc.exact_round_f32(mx - mn) / qmax)
        d16 = enc.exact_round_f16(d32)
        m16 = enc.exact_round_f16(mn)
        if isinstance(d16, float) or isinstance(m16, float):
            raise QuantRangeError("fp16 overflow")
        codes = []
        for w in vals:
            if d16 == 0:
                codes.append(0)
                continue
            num = enc.exact_round_f64(w - m16)
            q = _rint_half_even(enc.exact_round_f64(num / d16))
            codes.append(min(max(q, 0), qmax))
        return codes, (enc.exact_f16_bits(d16), enc.exact_f16_bits(m16, negative=(mn < 0 and m16 == 0)))
    if fmt == "int8":
        amax = max(abs(v) for v in vals)
        d16 = enc.exact_round_f16(enc.exact_round_f32(amax / 127))
        if isinstance(d16, float):
            raise QuantRangeError("fp16 overflow")
        codes = []
        for w in vals:
            if d16 == 0:
                codes.append(0)
                continue
            q = _rint_half_even(enc.exact_round_f64(w / d16))
            codes.append(min(max(q, -127), 127))
        return codes, (enc.exact_f16_bits(d16),)
    if fmt == "nvfp4":
        stf = Fraction(st)
        amax_b = max(abs(v) for v in vals)
        denom = enc.exact_round_f32(6 * stf)
        ratio = enc.exact_round_f32(amax_b / denom)
        sb = enc.exact_round_e4m3_sat(ratio)
        sb_code = enc.exact_e4m3_bits(sb)
        codes = []
        for w in vals:
            if sb == 0:
                codes.append(0)
                continue
            scale = enc.exact_round_f64(sb * stf)
            v = enc.exact_round_f64(w / scale)
            r = enc.exact_round_e2m1_sat(v)
            codes.append(enc.exact_e2m1_bits(r, negative=(w < 0)))
        return codes, (sb_code,)
    raise ValueError(fmt)


def nvfp4_tensor_scale_exact(W_values: list[float]) -> float:
    """s_t in exact arithmetic: fp32(amax / 2688), or 1 when that is zero."""
    amax = max(abs(Fraction(w)) for w in W_values)
    st = enc.exact_round_f32(amax / 2688)
    return 1.0 if st == 0 else float(st)
