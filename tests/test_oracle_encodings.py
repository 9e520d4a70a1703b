"""Pins for the oracle's number codecs: closed forms, exhaustive tables,
brute force in exact rationals and hand-derived golden values."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import encodings as enc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _same(a, b):
    if isinstance(a, float) and math.isnan(a):
        return isinstance(b, float) and math.isnan(b)
    return float(a) == float(b) and math.copysign(1, float(a)) == math.copysign(1, float(b))


def test_fp16_decode_exhaustive_matches_field_definition():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vec = enc.f64_from_f16_bits(bits)
    for b in range(65536):
        ex = enc.exact_f16_value(b)
        v = vec[b]
        if isinstance(ex, float):
            if math.isnan(ex):
                assert math.isnan(v)
            else:
                assert v == ex
        else:
            assert Fraction(float(v)) == ex
            if ex == 0:
                assert math.copysign(1, v) == (-1 if b & 0x8000 else 1)


def test_bf16_decode_exhaustive_matches_field_definition():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vec = enc.f32_from_bf16_bits(bits).astype(np.float64)
    for b in range(0, 65536):
        ex = enc.exact_bf16_value(b)
        v = vec[b]
        if isinstance(ex, float):
            assert (math.isnan(ex) and math.isnan(v)) or v == ex
        else:
            assert Fraction(float(v)) == ex


def _f16_probe_values():
    """All fp16 values, the midpoints between neighbours (ties), points just
    either side of each midpoint, overflow edges and random fp32 values."""
    pos = enc.f64_from_f16_bits(np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16))
    mids = (pos[:-1] + pos[1:]) / 2.0
    mids32 = mids.astype(np.float32)
    vals = [pos.astype(np.float32), mids32,
            np.nextafter(mids32, np.float32(np.inf)), np.nextafter(mids32, np.float32(0)),
            np.array([65504.0, 65519.0, 65519.996, 65520.0, 65536.0, 1e30, 2.0 ** -25,
                      2.0 ** -26, 3 * 2.0 ** -26, 1e-30], dtype=np.float32),
            np.random.default_rng(5).standard_normal(20000).astype(np.float32) * np.float32(30.0)]
    v = np.concatenate(vals)
    return np.concatenate([v, -v])


def test_fp16_encode_matches_exact_rounding():
    v = _f16_probe_values()
    got = enc.f16_bits_from_f32(v)
    # every probe, checked against the textbook rounding in rationals
    rng = np.random.default_rng(0)
    idx = np.concatenate([np.arange(0, v.size, 7), rng.integers(0, v.size, 3000)])
    for i in idx:
        x = float(v[i])
        r = enc.exact_round_f16(Fraction(x))
        want = enc.exact_f16_bits(r, negative=(x < 0 or (x == 0 and math.copysign(1, x) < 0)))
        assert int(got[i]) == want, (x, hex(int(got[i])), hex(want))


def test_fp16_ties_go_to_even():
    # 1 + 2^-11 lies halfway between 1 and 1 + 2^-10: even mantissa (1.0) wins
    assert enc.exact_round_f16(1 + Fraction(1, 2048)) == 1
    assert enc.exact_round_f16(1 + Fraction(3, 2048)) == 1 + Fraction(2, 1024)
    assert int(enc.f16_bits_from_f32(np.float32(1 + 2.0 ** -11))) == 0x3C00
    assert int(enc.f16_bits_from_f32(np.float32(1 + 3 * 2.0 ** -11))) == 0x3C02
    assert int(enc.f16_bits_from_f32(np.float32(65520.0))) == 0x7C00


def test_e4m3_table_closed_form_and_golden():
    g = _gold("scalar_values.json")["e4m3"]
    for code, want in g.items():
        v = enc.E4M3_TABLE[int(code)]
        if want == "nan":
            assert math.isnan(v)
        else:
            assert v == want
    # closed form: normals (8+m) 2^(e-10), subnormals m 2^-9, one NaN per sign
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            assert math.isnan(enc.E4M3_TABLE[b])
            continue
        mag = m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10)
        assert enc.E4M3_TABLE[b] == (-mag if s else mag)
    assert np.nanmax(enc.E4M3_TABLE) == 448.0


def test_e2m1_table_golden():
    g = _gold("scalar_values.json")["e2m1"]
    for c in range(16):
        assert _same(enc.E2M1_TABLE[c], g[c])


def _brute_nearest(v: Fraction, table):
    """Nearest finite table entry (ties -> even code) by full search."""
    best = None
    for code, t in table:
        d = abs(Fraction(t) - v)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


def test_e4m3_encoder_brute_force():
    table = [(c, enc.E4M3_TABLE[c]) for c in range(127)]
    rng = np.random.default_rng(1)
    pos = enc.E4M3_TABLE[:127]
    mids = (pos[:-1] + pos[1:]) / 2
    probes = np.concatenate([pos, mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
                             np.exp(rng.uniform(-16, 7, 3000)), [448.0, 460.0, 464.0, 470.0, 1e6, 0.0]])
    probes = probes.astype(np.float32)
    got = enc.e4m3_encode_sat(probes)
    for v, c in zip(probes, got):
        want = _brute_nearest(Fraction(float(v)), table)
        assert int(c) == want, (float(v), int(c), want)
        # and the exact rounding function agrees
        assert Fraction(enc.E4M3_TABLE[want]) == enc.exact_round_e4m3_sat(Fraction(float(v)))


def test_e2m1_encoder_brute_force_and_ties():
    table = [(c, enc.E2M1_TABLE[c]) for c in range(8)]
    g = _gold("scalar_values.json")["e2m1_round"]
    for v, want in g.items():
        c = int(enc.e2m1_encode_sat(np.array([float(v)]))[0])
        assert enc.E2M1_TABLE[c] == want
        c = int(enc.e2m1_encode_sat(np.array([-float(v)]))[0])
        assert enc.E2M1_TABLE[c] == -want or (want == 0 and c == 8)
    rng = np.random.default_rng(2)
    probes = np.concatenate([rng.uniform(-8, 8, 4000), np.arange(-7, 7.01, 0.125)])
    got = enc.e2m1_encode_sat(probes)
    for v, c in zip(probes, got):
        want = _brute_nearest(abs(Fraction(float(v))), table)
        assert int(c) & 7 == want
        assert (int(c) >> 3) == (1 if v < 0 else 0)


def test_e4m3_golden_rounding():
    g = _gold("scalar_values.json")["e4m3_round"]
    for v, want in g.items():
        c = int(enc.e4m3_encode_sat(np.array([float(v)], dtype=np.float32))[0])
        assert enc.E4M3_TABLE[c] == want, (v, c)


def test_fp16_golden():
    for b, want in _gold("scalar_values.json")["fp16"].items():
        assert float(enc.f64_from_f16_bits(np.array([int(b)], dtype=np.uint16))[0]) == want


def test_exact_encoders_roundtrip_all_codes():
    for b in range(256):
        v = enc.exact_e4m3_value(b)
        if isinstance(v, float):
            continue
        if v == 0:
            continue
        assert enc.exact_e4m3_bits(v) == b
    for b in range(16):
        v = enc.exact_e2m1_value(b)
        assert enc.exact_e2m1_bits(v, negative=bool(b & 8)) == b
    for b in range(0, 0x7C00, 13):
        v = enc.exact_f16_value(b)
        assert enc.exact_f16_bits(v) == b


@pytest.mark.parametrize("fn,p", [(enc.exact_round_f32, 24), (enc.exact_round_f64, 53)])
def test_exact_round_matches_hardware_float(fn, p):
    rng = np.random.default_rng(3)
    if p == 53:
        # Python's int / int true division is correctly rounded to double
        for _ in range(300):
            a = Fraction(int(rng.integers(1, 2 ** 62)), int(rng.integers(1, 2 ** 62)))
            a *= Fraction(2) ** int(rng.integers(-40, 40))
            assert fn(a) == Fraction(a.numerator / a.denominator)
        return
    # fp32: exact doubles (every one a Fraction exactly), rounded by numpy's
    # double -> float32 cast, which rounds to nearest even (IEEE 754)
    samples = []
    for _ in range(300):                        # random doubles across the fp32 range, subnormals included
        m = int(rng.integers(2 ** 52, 2 ** 53))
        samples.append(math.ldexp(m, int(rng.integers(-52 - 150, -52 + 128))))
    for _ in range(100):                        # exact ties between neighbouring fp32 values
        f = np.float32(rng.standard_normal() * 2.0 ** int(rng.integers(-130, 120)))
        nxt = np.nextafter(f, np.float32(np.inf))
        samples.append((float(f) + float(nxt)) / 2)
    for d in samples:
        for v in (d, -d):
            want = Fraction(float(np.float32(v))) if abs(v) < float(np.finfo(np.float32).max) else None
            if want is None or not math.isfinite(float(np.float32(v))):
                continue
            assert fn(Fraction(v)) == want, v
