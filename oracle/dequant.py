"""Dequantisation: logical fields -> fp32 weights (oracle; test infrastructure).

This is the definition the GPU's debug dump must match bit for bit:
  * asymmetric int4 / int5:  w = RN32(d * q + m)
    (d * q is exact, so the value is one rounding of the exact sum; in fp64
    both terms are multiples of 2^-24 below 2^22, so the fp64 sum is exact
    and the final cast is the only rounding);
  * symmetric int8:          w = d * q (exact in fp32);
  * NVFP4:                   w = RN32(s_t * (e2m1(code) * e4m3(scale)))
    (the inner product has at most 6 significant bits, the full product at
    most 30, so fp64 holds it exactly and the cast is the only rounding);
  * MXFP8 / MXFP4:           w = e4m3(code) * 2^(e - 127) or
                             e2m1(code) * 2^(e - 127), exact in fp32 (at most 4
    significant bits; X >= -127 keeps every product at or above 2^-136, a
    multiple of fp32's 2^-149 step, and X <= 119 keeps it below 2^128).
Formats per the NInfer article (section 2: groupwise int Q4/Q5 and NVFP4
weights), the RustingStrata page (Q8_0-style int8) and the Decapybara page
(NVFP4 blocked GEMV, MXFP8 block-scaled GEMV).
"""
from __future__ import annotations

import numpy as np

from . import encodings as enc
from .quant import Quantized, GROUP, MX_BLOCK, NVFP4_BLOCK


def dequant(qz: Quantized) -> np.ndarray:
    """Return the fp32 [M][K] weights that the codes and scales encode."""
    M, K = qz.M, qz.K
    if qz.fmt in ("int4", "int5"):
        d = np.repeat(enc.f64_from_f16_bits(qz.d), GROUP, axis=1)
        m = np.repeat(enc.f64_from_f16_bits(qz.m), GROUP, axis=1)
        with np.errstate(invalid="ignore", over="ignore"):
            return (d * qz.codes.astype(np.float64) + m).astype(np.float32)
    if qz.fmt == "int8":
        d = np.repeat(enc.f64_from_f16_bits(qz.d), GROUP, axis=1)
        with np.errstate(invalid="ignore", over="ignore"):
            return (d * qz.codes.astype(np.float64)).astype(np.float32)
    if qz.fmt == "nvfp4":
        sb = np.repeat(enc.e4m3_decode(qz.sb), NVFP4_BLOCK, axis=1)
        v = enc.e2m1_decode(qz.codes) * sb
        with np.errstate(invalid="ignore", over="ignore"):
            return (np.float64(qz.st) * v).astype(np.float32)
    if qz.fmt in ("mxfp8", "mxfp4"):
        sc = np.repeat(enc.e8m0_decode(qz.e), MX_BLOCK, axis=1)
        v = enc.e4m3_decode(qz.codes) if qz.fmt == "mxfp8" else enc.e2m1_decode(qz.codes)
        return (v * sc).astype(np.float32)
    raise ValueError(qz.fmt)
