"""Pins for the oracle's quantisers, layout and dequantisation: exact
rational re-derivation of every group, brute-force nearest codes, exact
round trips of representable groups, hand-derived bytes and values."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synthetic
from oracle import encodings as enc
from oracle import layout, quant
from oracle.dequant import dequant

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FORMATS = ["int4", "int5", "int8", "nvfp4"]


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _adversarial_rows(K, rng):
    """Rows that stress the quantisers: constant, tiny, huge-range, signed
    extremes, a single outlier, exact zeros, fp16-subnormal scales."""
    rows = [
        np.full(K, 0.125, np.float32),
        np.zeros(K, np.float32),
        np.full(K, -3.0e-6, np.float32),
        (rng.standard_normal(K) * 1e-7).astype(np.float32),
        (rng.standard_normal(K) * 100).astype(np.float32),
        np.where(np.arange(K) % 32 == 7, 5.0, 0.0).astype(np.float32),
        np.where(np.arange(K) % 2 == 0, 1.0, -1.0).astype(np.float32),
        np.linspace(-1, 1, K).astype(np.float32),
        (rng.standard_normal(K) * 0.02).astype(np.float32),
    ]
    return np.stack(rows)


@pytest.mark.parametrize("fmt", FORMATS)
def test_vectorised_quantiser_matches_exact_rational(fmt):
    rng = np.random.default_rng(11)
    K = 64
    W = np.concatenate([_adversarial_rows(K, rng), synthetic.weights(rng, 6, K)])
    qz = quant.quantize(W, fmt)
    if fmt == "nvfp4":
        st = quant.nvfp4_tensor_scale_exact([float(v) for v in W.reshape(-1)])
        assert np.float32(st) == qz.st
        for m in range(W.shape[0]):
            for b in range(K // 16):
                ws = [float(v) for v in W[m, 16 * b: 16 * b + 16]]
                codes, (sb,) = quant.quantize_group_exact(ws, fmt, st=st)
                assert int(qz.sb[m, b]) == sb
                got = [int(c) for c in qz.codes[m, 16 * b: 16 * b + 16]]
                # the sign of a zero code is the sign of its weight in both
                assert got == codes, (m, b, got, codes)
        return
    for m in range(W.shape[0]):
        for g in range(K // 32):
            ws = [float(v) for v in W[m, 32 * g: 32 * g + 32]]
            codes, fields = quant.quantize_group_exact(ws, fmt)
            assert [int(c) for c in qz.codes[m, 32 * g: 32 * g + 32]] == codes
            assert int(qz.d[m, g]) == fields[0]
            if fmt != "int8":
                assert int(qz.m[m, g]) == fields[1]


@pytest.mark.parametrize("fmt", ["int4", "int5", "int8"])
def test_int_codes_are_nearest_by_brute_force(fmt):
    rng = np.random.default_rng(12)
    W = np.concatenate([_adversarial_rows(32, rng), synthetic.weights(rng, 20, 32)])
    qz = quant.quantize(W, fmt)
    lo, hi = (-127, 127) if fmt == "int8" else (0, 15 if fmt == "int4" else 31)
    for m in range(W.shape[0]):
        d = Fraction(float(enc.f64_from_f16_bits(qz.d[m:m + 1, 0])[0]))
        mm = Fraction(0) if fmt == "int8" else Fraction(float(enc.f64_from_f16_bits(qz.m[m:m + 1, 0])[0]))
        for k in range(32):
            w = Fraction(float(W[m, k]))
            q = int(qz.codes[m, k])
            if d == 0:
                assert q == 0
                continue
            err = abs(w - (d * q + mm))
            best = min(abs(w - (d * c + mm)) for c in range(lo, hi + 1))
            # fp64 quotient rounding may only matter at an exact tie
            assert err <= best + d * Fraction(1, 2 ** 40), (m, k, q)


def test_nvfp4_codes_are_nearest_by_brute_force():
    rng = np.random.default_rng(13)
    W = synthetic.weights(rng, 8, 64)
    qz = quant.quantize(W, "nvfp4")
    st = Fraction(float(qz.st))
    for m in range(8):
        for k in range(64):
            sb = Fraction(float(enc.E4M3_TABLE[qz.sb[m, k // 16]]))
            w = Fraction(float(W[m, k]))
            got = Fraction(float(enc.E2M1_TABLE[qz.codes[m, k]])) * sb * st
            best = min(abs(w - Fraction(float(enc.E2M1_TABLE[c])) * sb * st) for c in range(16))
            assert abs(w - got) <= best * (1 + Fraction(1, 2 ** 40))


def test_representable_groups_round_trip_exactly():
    """Quantise(dequant(fields)) == fields when the arithmetic is exact:
    power-of-two d and m, codes spanning both ends of the range."""
    rng = np.random.default_rng(14)
    for fmt, qmax in (("int4", 15), ("int5", 31)):
        codes = rng.integers(0, qmax + 1, size=(4, 64)).astype(np.uint8)
        codes[:, 0] = 0
        codes[:, 31] = qmax
        codes[:, 32] = qmax
        codes[:, 63] = 0
        d = np.float32(2.0 ** -5)
        m = np.float32(-0.5)
        W = (d * codes.astype(np.float32) + m).astype(np.float32)
        qz = quant.quantize(W, fmt)
        assert np.array_equal(qz.codes, codes)
        assert np.all(qz.d == enc.f16_bits_from_f32(np.float32(d)))
        assert np.all(qz.m == enc.f16_bits_from_f32(m))
    codes = rng.integers(-127, 128, size=(4, 64)).astype(np.int8)
    codes[:, 5] = 127
    codes[:, 40] = -127
    W = (np.float32(2.0 ** -6) * codes.astype(np.float32)).astype(np.float32)
    qz = quant.quantize(W, "int8")
    assert np.array_equal(qz.codes, codes)
    assert np.all(qz.d == 0x2400)
    # nvfp4: s_t = 2^-10 (amax = 2688 * 2^-10), block scales from E4M3 values
    sb_codes = rng.integers(0x30, 0x7F, size=(4, 4)).astype(np.uint8)
    sb_codes[0, 0] = 0x7E                          # 448: the matrix maximum
    e2 = rng.integers(0, 16, size=(4, 64)).astype(np.uint8)
    e2[:, ::16] = 7                                # each block reaches +6
    e2[e2 == 8] = 0                                # no negative zeros
    st = np.float32(2.0 ** -10)
    vals = enc.E2M1_TABLE[e2] * np.repeat(enc.E4M3_TABLE[sb_codes], 16, axis=1) * float(st)
    W = vals.astype(np.float32)
    qz = quant.quantize(W, "nvfp4")
    assert qz.st == st
    assert np.array_equal(qz.sb, sb_codes)
    assert np.array_equal(qz.codes, e2)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,K", [(16, 128), (17, 160), (1, 32), (33, 512), (5, 96)])
def test_pack_unpack_round_trip(fmt, M, K):
    rng = np.random.default_rng(M * 1000 + K)
    if fmt == "int8":
        codes = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    else:
        codes = rng.integers(0, {"int4": 16, "int5": 32, "nvfp4": 16}[fmt], size=(M, K)).astype(np.uint8)
    qz = quant.Quantized(fmt, M, K, codes)
    if fmt == "nvfp4":
        qz.sb = rng.integers(0, 256, size=(M, K // 16)).astype(np.uint8)
        qz.st = np.float32(rng.standard_normal())
    else:
        qz.d = rng.integers(0, 65536, size=(M, K // 32)).astype(np.uint16)
        if fmt != "int8":
            qz.m = rng.integers(0, 65536, size=(M, K // 32)).astype(np.uint16)
    wq, ws = layout.pack(qz)
    assert (wq.size, ws.size) == layout.packed_bytes(fmt, M, K)
    back = layout.unpack(fmt, M, K, wq, ws)
    assert np.array_equal(back.codes, qz.codes)
    if fmt == "nvfp4":
        assert np.array_equal(back.sb, qz.sb) and back.st == qz.st
    else:
        assert np.array_equal(back.d, qz.d)
        if fmt != "int8":
            assert np.array_equal(back.m, qz.m)


def test_packed_sizes_match_bits_per_weight():
    M, K = 17408, 5120
    assert sum(layout.packed_bytes("int4", M, K)) == M * K * 5 // 8
    assert sum(layout.packed_bytes("int5", M, K)) == M * K * 6 // 8
    assert sum(layout.packed_bytes("int8", M, K)) == M * K * 17 // 16
    assert sum(layout.packed_bytes("nvfp4", M, K)) == M * K * 9 // 16 + 16


def test_int4_golden_block_bytes_and_values():
    g = _gold("int4_block.json")
    qz = quant.Quantized("int4", g["M"], g["K"], np.array([g["codes"]], np.uint8),
                         d=np.array([[g["d_bits"]]], np.uint16), m=np.array([[g["m_bits"]]], np.uint16))
    wq, ws = layout.pack(qz)
    expect = np.zeros_like(wq)
    for off, b in g["wq_bytes_at"].items():
        expect[int(off): int(off) + len(b)] = b
    assert np.array_equal(wq, expect)
    for off, b in g["ws_bytes_at"].items():
        assert list(ws[int(off): int(off) + len(b)]) == b
    assert np.count_nonzero(ws) == 2
    w = dequant(qz)
    assert list(w[0]) == g["values"]
    # and quantising the golden values reproduces the golden fields
    q2 = quant.quantize(w.astype(np.float32), "int4")
    assert np.array_equal(q2.codes, qz.codes) and q2.d[0, 0] == g["d_bits"] and q2.m[0, 0] == g["m_bits"]


def test_dequant_golden_values():
    g = _gold("scalar_values.json")["dequant"]
    c = np.zeros((1, 32), np.uint8)
    c[0, 0] = g["int5"]["code"]
    qz = quant.Quantized("int5", 1, 32, c, d=np.array([[g["int5"]["d_bits"]]], np.uint16),
                         m=np.array([[g["int5"]["m_bits"]]], np.uint16))
    assert dequant(qz)[0, 0] == g["int5"]["value"]
    c = np.zeros((1, 32), np.int8)
    c[0, :5] = g["int8"]["codes"]
    qz = quant.Quantized("int8", 1, 32, c, d=np.array([[g["int8"]["d_bits"]]], np.uint16))
    assert list(dequant(qz)[0, :5]) == g["int8"]["values"]
    c = np.zeros((1, 32), np.uint8)
    c[0, 3] = g["nvfp4"]["code"]
    qz = quant.Quantized("nvfp4", 1, 32, c, sb=np.full((1, 2), g["nvfp4"]["sb"], np.uint8),
                         st=np.float32(g["nvfp4"]["st"]))
    assert dequant(qz)[0, 3] == g["nvfp4"]["value"]


@pytest.mark.parametrize("fmt", FORMATS)
def test_dequant_is_one_exact_rounding(fmt):
    """Every dequantised value equals the exact rational value rounded once."""
    rng = np.random.default_rng(21)
    M, K = 4, 64
    if fmt == "int8":
        codes = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    else:
        codes = rng.integers(0, 32 if fmt == "int5" else 16, size=(M, K)).astype(np.uint8)
    # fp16 fields over the whole finite range, including subnormals
    finite16 = np.array([b for b in range(0, 0x7C00, 37)] + [b | 0x8000 for b in range(0, 0x7C00, 41)], np.uint16)
    qz = quant.Quantized(fmt, M, K, codes)
    if fmt == "nvfp4":
        fin = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
        qz.sb = rng.choice(fin, size=(M, K // 16)).astype(np.uint8)
        qz.st = np.float32(3.1e-3)
    else:
        qz.d = rng.choice(finite16, size=(M, K // 32))
        if fmt != "int8":
            qz.m = rng.choice(finite16, size=(M, K // 32))
    w = dequant(qz)
    for m in range(M):
        for k in range(K):
            if fmt == "nvfp4":
                exact = (enc.exact_e2m1_value(int(codes[m, k])) * enc.exact_e4m3_value(int(qz.sb[m, k // 16]))
                         * Fraction(float(qz.st)))
            else:
                d = enc.exact_f16_value(int(qz.d[m, k // 32]))
                exact = d * int(codes[m, k])
                if fmt != "int8":
                    exact += enc.exact_f16_value(int(qz.m[m, k // 32]))
            r = enc.exact_round_f32(exact)
            assert Fraction(float(w[m, k])) == r, (fmt, m, k)


def test_layout_spot_bytes_golden():
    """One nonzero field at a time lands on the hand-derived byte."""
    g = _gold("layout_spots.json")
    M, K = g["M"], g["K"]
    for case in g["cases"]:
        fmt = case["fmt"]
        codes = np.zeros((M, K), np.int8 if fmt == "int8" else np.uint8)
        qz = quant.Quantized(fmt, M, K, codes)
        if fmt == "nvfp4":
            qz.sb = np.zeros((M, K // 16), np.uint8)
            qz.st = np.float32(0.0)
        else:
            qz.d = np.zeros((M, K // 32), np.uint16)
            qz.m = None if fmt == "int8" else np.zeros((M, K // 32), np.uint16)
        if "code" in case:
            codes[case["m"], case["k"]] = case["code"]
            want, key = case["wq"], 0
        elif "sb" in case:
            qz.sb[case["m"], case["b"]] = case["sb"]
            want, key = case["ws"], 1
        else:
            qz.d[case["m"], case["g"]] = case["d_bits"]
            if "m_bits" in case:
                qz.m[case["m"], case["g"]] = case["m_bits"]
            want, key = case["ws"], 1
        buf = layout.pack(qz)[key]
        expect = np.zeros_like(buf)
        for off, v in want.items():
            expect[int(off)] = v
        assert np.array_equal(buf, expect), (case, np.nonzero(buf)[0], buf[np.nonzero(buf)[0]])
