"""Pins of the oracle's MX (microscaling) formats: E8M0 scales, MXFP8 / MXFP4
quantisation, the activation quantiser, dequantisation and the layout.

The Decapybara kernel list names an MXFP8 block-scaled GEMV and a dynamic
32-element MXFP8 activation quantiser without defining them; the pins come
from the public OCP definitions: hand-worked blocks (tests/golden), closed
forms, brute force over every code, and error bounds.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import dequant as D
from oracle import encodings as enc
from oracle import layout as L
from oracle import quant as Q

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits_to_f32(bits):
    return np.array([int(b, 16) for b in bits], dtype=np.uint32).view(np.float32)


def test_e8m0_closed_form():
    assert enc.E8M0_TABLE[127] == 1.0
    assert enc.E8M0_TABLE[128] == 2.0
    assert enc.E8M0_TABLE[0] == 2.0 ** -127
    assert enc.E8M0_TABLE[254] == 2.0 ** 127
    assert math.isnan(enc.E8M0_TABLE[255])
    for b in range(255):
        assert enc.E8M0_TABLE[b] == math.ldexp(1.0, b - 127)
        assert enc.exact_e8m0_value(b) == Fraction(2) ** (b - 127)


def test_mx_golden_blocks():
    d = json.load(open(os.path.join(GOLD, "mx_blocks.json")))
    assert len(d["blocks"]) >= 8
    for b in d["blocks"]:
        vals = _bits_to_f32(b["bits"] + [b["fill"]] * (32 - len(b["bits"])))
        want = b["codes"] + [b["fill_code"]] * (32 - len(b["codes"]))
        codes, e = Q.mx_quantize_blocks(vals.reshape(1, 32), b["fmt"])
        assert list(codes[0]) == want, b["why"]
        assert int(e[0]) == b["scale_byte"], b["why"]
        ce, ee = Q.mx_block_exact([float(v) for v in vals], b["fmt"])
        assert ce == want and ee == b["scale_byte"], b["why"]


def _brute_code(v: float, fmt: str) -> int:
    """Nearest finite code by exhaustive search (ties: even code), the sign
    taken from v; magnitudes past the largest finite value saturate."""
    table = enc.E4M3_TABLE if fmt == "mxfp8" else enc.E2M1_TABLE
    sign_bit = 0x80 if fmt == "mxfp8" else 0x8
    neg = math.copysign(1.0, v) < 0
    best, best_d = None, None
    for c in range(len(table)):
        val = table[c]
        if math.isnan(val) or bool(c & sign_bit) != neg:
            continue
        dist = abs(abs(v) - abs(val))
        if best is None or dist < best_d or (dist == best_d and c % 2 == 0 and best % 2 == 1):
            best, best_d = c, dist
    return best


def _brute_scale(amax: float, emax: int) -> int:
    if amax == 0:
        return -127
    e = 0
    while math.ldexp(1.0, e) > amax:
        e -= 1
    while math.ldexp(1.0, e + 1) <= amax:
        e += 1
    return max(-127, min(127, e - emax))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_brute_force(fmt):
    rng = np.random.default_rng(5)
    for trial in range(24):
        mag = math.exp(rng.uniform(-100, 80))
        V = (rng.standard_normal(32) * mag).astype(np.float32)
        if trial % 6 == 0:
            V[rng.integers(0, 32, 5)] = 0.0
        if trial % 8 == 1:
            V[3] = -0.0
        codes, e = Q.mx_quantize_blocks(V.reshape(1, 32), fmt)
        X = _brute_scale(float(np.abs(V.astype(np.float64)).max()), Q.MX_EMAX[fmt])
        assert int(e[0]) == X + 127
        for i in range(32):
            assert int(codes[0, i]) == _brute_code(float(V[i]) / 2.0 ** X, fmt), (trial, i, V[i])


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_error_bound_and_dequant(fmt):
    """Every element is within half a step of its binade (E4M3: 2^-4, E2M1:
    2^-2 relative) or half the least subnormal step, unless it saturated;
    the block maximum lands in the element format's top binade before
    rounding; dequant = value(code) * 2^X exactly."""
    rng = np.random.default_rng(6)
    W = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-40, 40, (64, 1)))).astype(np.float32)
    qz = Q.quantize(W, fmt)
    Wd = D.dequant(qz).astype(np.float64)
    X = qz.e.astype(np.int64) - 127
    sc = np.repeat(np.ldexp(1.0, X), 32, axis=1)
    rel, sub = (2.0 ** -4, 2.0 ** -10) if fmt == "mxfp8" else (2.0 ** -2, 2.0 ** -2)
    top = 448.0 if fmt == "mxfp8" else 6.0
    w = W.astype(np.float64)
    sat = np.abs(w) / sc > top
    err = np.abs(Wd - w)
    assert np.all(err[~sat] <= rel * np.abs(w[~sat]) + sub * sc[~sat])
    assert np.all(np.abs(Wd[sat]) == top * sc[sat])
    amax = np.abs(w.reshape(64, -1, 32)).max(axis=2)
    ratio = amax / np.ldexp(1.0, X)
    emax = Q.MX_EMAX[fmt]
    assert np.all((ratio >= 2.0 ** emax) & (ratio < 2.0 ** (emax + 1)))
    vals = enc.e4m3_decode(qz.codes) if fmt == "mxfp8" else enc.e2m1_decode(qz.codes)
    assert np.array_equal(Wd, vals * sc)


def test_act_quant_matches_exact_blocks_and_keeps_zero_sign():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((3, 96)) * np.array([[1e-3], [1.0], [3e4]])).astype(np.float32)
    x[0, 0] = -0.0
    x[1, 32:64] = 0.0
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)      # truncation to bf16 is fine for a pin input
    codes, e = Q.mx_act_quant(bits)
    xf = enc.f32_from_bf16_bits(bits)
    for n in range(3):
        for b in range(3):
            ce, ee = Q.mx_block_exact([float(v) for v in xf[n, 32 * b:32 * b + 32]], "mxfp8")
            assert list(codes[n, 32 * b:32 * b + 32]) == ce and int(e[n, b]) == ee
    assert codes[0, 0] == 0x80
    assert e[1, 1] == 0 and not codes[1, 32:64].any()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("M,K", [(16, 128), (37, 160), (5, 32), (48, 640)])
def test_mx_layout_round_trip_and_spots(fmt, M, K):
    rng = np.random.default_rng(M * K)
    W = rng.standard_normal((M, K)).astype(np.float32)
    qz = Q.quantize(W, fmt)
    wq, ws = L.pack(qz)
    assert (wq.size, ws.size) == L.packed_bytes(fmt, M, K)
    back = L.unpack(fmt, M, K, wq, ws)
    assert np.array_equal(back.codes, qz.codes) and np.array_equal(back.e, qz.e)
    # spot bytes from the layout specification, tile (rt, ks) = (0, 0)
    for lam, i in ((0, 0), (37, 5), (63, 15)):
        r, g = lam % 16, lam // 16
        if r >= M:
            continue
        if fmt == "mxfp8":
            for h in (0, 1):
                k = 64 * h + 16 * g + i
                assert wq[h * 1024 + lam * 16 + i] == (qz.codes[r, k] if k < K else 0)
        else:
            k = 32 * g + 2 * i
            lo = qz.codes[r, k] if k < K else 0
            hi = qz.codes[r, k + 1] if k + 1 < K else 0
            assert wq[lam * 16 + i] == (lo | (hi << 4))
        assert ws[lam] == (qz.e[r, g] if 32 * g < K else 0)


def test_mx_activations_definition():
    """The MX GEMV's activations are the dequantised MXFP8 codes: closed form
    on a block whose values are exactly representable (no rounding)."""
    from oracle import gemv as G
    v = np.array([1.0, -0.5, 3.0, 0.25] * 8, dtype=np.float32).reshape(1, 32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(G.mx_activations(bits), v.astype(np.float64))
