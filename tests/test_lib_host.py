"""CPU tests of the C-ABI library: exported symbols, host packer bytes against
the oracle's packer, and argument validation (no GPU call is ever reached)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synthetic
from oracle import layout, quant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
qg = pytest.importorskip("bit_quantized_weight_amd")
if not os.path.exists(qg.LIB_PATH):
    pytest.skip("libqgemv.so not built (run __graft_entry__.build())", allow_module_level=True)

FORMATS = ["int4", "int5", "int8", "nvfp4", "mxfp4", "mxfp8"]


def _header_functions():
    src = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemv[a-z_]*)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = qg.load(False)
    declared = _header_functions()
    assert len(declared) >= 13
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(qg.symbols()) == declared


def test_version_and_strerror():
    assert qg.load(False).qgemv_version() >= 100
    for code in range(0, -8, -1):
        assert len(qg.strerror(code)) > 3
    assert qg.strerror(-99) == "unknown status"


def _rows(K, rng):
    rows = [np.zeros(K), np.full(K, 0.125), np.linspace(-1, 1, K), rng.standard_normal(K) * 1e-6,
            rng.standard_normal(K) * 3, np.where(np.arange(K) % 32 == 3, -5.0, 0.0), -np.zeros(K)]
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,K", [(16, 128), (23, 160), (1, 32), (40, 640), (7, 96)])
def test_pack_bytes_equal_oracle(fmt, M, K):
    rng = np.random.default_rng(M * 131 + K)
    W = synthetic.weights(rng, M, K)
    W[: min(M, 7)] = _rows(K, rng)[: min(M, 7)]
    wq, ws = qg.pack(fmt, W)
    owq, ows = layout.pack(quant.quantize(W, fmt))
    assert wq.size == owq.size and ws.size == ows.size
    assert np.array_equal(wq, owq), np.nonzero(wq != owq)[0][:10]
    assert np.array_equal(ws, ows), np.nonzero(ws != ows)[0][:10]


@pytest.mark.parametrize("fmt", FORMATS)
def test_pack_bytes_equal_oracle_large(fmt):
    rng = np.random.default_rng(99)
    W = synthetic.weights(rng, 512, 5120)
    wq, ws = qg.pack(fmt, W)
    owq, ows = layout.pack(quant.quantize(W, fmt))
    assert np.array_equal(wq, owq) and np.array_equal(ws, ows)


@pytest.mark.parametrize("fmt", FORMATS)
def test_pack_codes_equal_oracle(fmt):
    rng = np.random.default_rng(5)
    M, K = 33, 384
    hi = {"int4": 16, "int5": 32, "nvfp4": 16, "mxfp4": 16, "mxfp8": 256}.get(fmt)
    codes = (rng.integers(-128, 128, (M, K)).astype(np.int8) if fmt == "int8"
             else rng.integers(0, hi, (M, K)).astype(np.uint8))
    if fmt == "mxfp8":
        codes[(codes & 0x7F) == 0x7F] = 0x7E          # E4M3 NaN codes are rejected
    qz = quant.Quantized(fmt, M, K, codes)
    if fmt in ("mxfp4", "mxfp8"):
        qz.e = rng.integers(0, 255, (M, K // 32)).astype(np.uint8)
        wq, ws = qg.pack_codes(fmt, codes, qz.e)
    elif fmt == "nvfp4":
        qz.sb = rng.integers(0, 256, (M, K // 16)).astype(np.uint8)
        qz.st = np.float32(0.37)
        wq, ws = qg.pack_codes(fmt, codes, qz.sb, None, float(qz.st))
    else:
        qz.d = rng.integers(0, 65536, (M, K // 32)).astype(np.uint16)
        qz.m = None if fmt == "int8" else rng.integers(0, 65536, (M, K // 32)).astype(np.uint16)
        wq, ws = qg.pack_codes(fmt, codes, qz.d, qz.m)
    owq, ows = layout.pack(qz)
    assert np.array_equal(wq, owq) and np.array_equal(ws, ows)


def test_pack_rejects_bad_input():
    W = np.zeros((16, 64), np.float32)
    with pytest.raises(qg.QgemvError) as e:
        qg.pack(9, W)
    assert e.value.status == -2
    Wn = W.copy()
    Wn[3, 4] = np.nan
    with pytest.raises(qg.QgemvError) as e:
        qg.pack("int4", Wn)
    assert e.value.status == -1
    big = np.full((16, 64), 1e7, np.float32)
    big[:, ::2] = -1e7
    for fmt in ("int4", "int5", "int8"):
        with pytest.raises(qg.QgemvError) as e:
            qg.pack(fmt, big)
        assert e.value.status == -4
    with pytest.raises(qg.QgemvError) as e:
        qg.packed_bytes("int4", 16, 48)
    assert e.value.status == -1
    codes = np.full((16, 64), 16, np.uint8)
    with pytest.raises(qg.QgemvError) as e:
        qg.pack_codes("int4", codes, np.zeros((16, 2), np.uint16), np.zeros((16, 2), np.uint16))
    assert e.value.status == -1


def test_pack_codes_rejects_mx_nan():
    codes = np.zeros((16, 64), np.uint8)
    e = np.full((16, 2), 127, np.uint8)
    codes[2, 5] = 0x7F
    with pytest.raises(qg.QgemvError) as ex:
        qg.pack_codes("mxfp8", codes, e)
    assert ex.value.status == -1
    codes[2, 5] = 0
    e[1, 1] = 0xFF
    with pytest.raises(qg.QgemvError) as ex:
        qg.pack_codes("mxfp8", codes, e)
    assert ex.value.status == -1


def test_expert_stride_is_256_aligned():
    a, b = qg.expert_stride("nvfp4", 1536, 2048)
    pa, pb = qg.packed_bytes("nvfp4", 1536, 2048)
    assert a % 256 == 0 and b % 256 == 0 and a >= pa and b >= pb and b - pb < 256


# Device entry points: every call below fails validation on the host, so no
# HIP call is made and these run without a GPU.
FAKE = 0x10000          # 16-byte aligned, never dereferenced
ODD = 0x10004


def _gemv(**kw):
    a = dict(fmt=1, wq=FAKE, ws=FAKE, x=FAKE, res=None, y=FAKE, M=64, K=128, N=1, stream=None)
    a.update(kw)
    return qg.load(False).qgemv(a["fmt"], a["wq"], a["ws"], a["x"], a["res"], a["y"], a["M"], a["K"], a["N"],
                                a["stream"])


def test_qgemv_validation_codes():
    assert _gemv(fmt=0) == -2 and _gemv(fmt=5) == -2
    assert _gemv(wq=None) == -1 and _gemv(x=None) == -1 and _gemv(y=None) == -1
    assert _gemv(N=0) == -7 and _gemv(N=33) == -7 and _gemv(fmt=4, N=33) == -7
    assert _gemv(K=48) == -3 and _gemv(K=0) == -1 and _gemv(M=0) == -1
    assert _gemv(wq=ODD) == -3 and _gemv(x=ODD) == -3 and _gemv(y=FAKE + 2) == -3
    assert _gemv(res=FAKE + 1, y=FAKE) == -3
    L = qg.load(False)
    assert L.qgemv_swiglu(1, FAKE, FAKE, FAKE, FAKE, 24, 128, 1, None) == -3      # I % 16
    assert L.qgemv_swiglu(1, FAKE, FAKE, FAKE, FAKE, 32, 128, 33, None) == -7
    assert L.qgemv_dequant(1, FAKE, FAKE, 16, 40, FAKE, None) == -3
    assert L.qgemv_dequant(7, FAKE, FAKE, 16, 64, FAKE, None) == -2
    assert L.qgemv_probe_read(FAKE, 100, FAKE, None) == -3
    assert L.qgemv_probe_read(None, 128, FAKE, None) == -1


def test_qgemv_moe_validation_codes():
    L = qg.load(False)
    need = qg.moe_workspace_bytes(128, 2048, 768, 8, 8)
    assert need > 0

    def moe(**kw):
        a = dict(fmt=1, E=128, H=2048, I=768, top_k=8, N=8, ws=FAKE, wsb=need, ids=FAKE)
        a.update(kw)
        return L.qgemv_moe(a["fmt"], FAKE, FAKE, FAKE, FAKE, a["E"], a["H"], a["I"], FAKE, a["ids"], FAKE,
                           a["top_k"], None, FAKE, a["N"], a["ws"], a["wsb"], None)
    assert moe(ws=None) == -5
    assert moe(wsb=need - 1) == -5
    assert moe(top_k=9) == -7 and moe(N=9) == -7
    assert moe(H=2047) == -1 or moe(H=2047) == -3
    assert moe(fmt=0) == -2
    assert moe(ids=None) == -1
    assert moe(E=16385) == -7          # routing bitmap limit: 16384 experts
    assert L.qgemv_moe_index(None, 1, 8, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert L.qgemv_moe_index(FAKE, 9, 8, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -7
    b = ctypes.c_size_t()
    assert L.qgemv_moe_workspace_bytes(0, 2048, 768, 1, 8, ctypes.byref(b)) == -1


def test_router_and_fused_moe_validation_codes():
    """Argument checks of qgemv_moe_route and qgemv_moe_fused return before
    any launch (no GPU needed)."""
    L = qg.load(False)
    assert L.qgemv_moe_route(None, 2, 8, 2, FAKE, FAKE, None) == -1
    assert L.qgemv_moe_route(FAKE, 2, 8, 9, FAKE, FAKE, None) == -7           # top_k > E
    assert L.qgemv_moe_route(FAKE, 2, 100, 65, FAKE, FAKE, None) == -7        # top_k > 64
    assert L.qgemv_moe_route(FAKE, 2, 16385, 8, FAKE, FAKE, None) == -7       # E limit
    assert L.qgemv_moe_route(FAKE + 2, 2, 8, 2, FAKE, FAKE, None) == -3
    need = qg.moe_fused_workspace_bytes(128, 2048, 768, 8, 8)
    assert need > qg.moe_workspace_bytes(128, 2048, 768, 8, 8)

    def fused(**kw):
        a = dict(fmt=1, E=128, H=2048, I=768, top_k=8, N=8, ws=FAKE, wsb=need, logits=FAKE)
        a.update(kw)
        return L.qgemv_moe_fused(a["fmt"], FAKE, FAKE, FAKE, FAKE, a["E"], a["H"], a["I"], FAKE, a["logits"],
                                 a["top_k"], None, FAKE, a["N"], None, None, a["ws"], a["wsb"], None)
    assert fused(ws=None) == -5 and fused(wsb=need - 1) == -5
    assert fused(logits=None) == -1 and fused(logits=FAKE + 2) == -3
    assert fused(top_k=9) == -7 and fused(N=9) == -7 and fused(E=4, top_k=5) == -7
    assert fused(fmt=9) == -2 and fused(H=2047) in (-1, -3)
    b = ctypes.c_size_t()
    assert L.qgemv_moe_fused_workspace_bytes(128, 2048, 768, 0, 8, ctypes.byref(b)) == -7


def test_fusion_validation_codes():
    """qgemv_ex / qgemv_swiglu_ex argument checks (before any launch)."""
    L = qg.load(False)

    def ex(x=FAKE, y=FAKE, src=None, gamma=None, eps=1e-6, ybf=None, M=64, K=128, N=1, sw=False, flags=0):
        fz = qg.Fusion(src, gamma, eps, ybf, flags)
        if sw:
            return L.qgemv_swiglu_ex(1, FAKE, FAKE, x, y, M, K, N, ctypes.byref(fz), None)
        return L.qgemv_ex(1, FAKE, FAKE, x, None, y, M, K, N, ctypes.byref(fz), None)
    assert ex(src=FAKE, gamma=None) == -1                 # gamma required with the prologue
    assert ex(src=FAKE + 4, gamma=FAKE) == -3              # 16-byte alignment of the source
    assert ex(src=FAKE, gamma=FAKE + 8) == -3
    assert ex(src=FAKE, gamma=FAKE, eps=-1.0) == -1
    assert ex(src=FAKE, gamma=FAKE, eps=float("nan")) == -1
    assert ex(x=None) == -1                                # no activations and no prologue
    assert ex(y=None, ybf=None) == -1                      # no output at all
    assert ex(y=None, ybf=FAKE + 1) == -3                  # bf16 output must be 2-byte aligned
    assert ex(N=9, src=FAKE, gamma=FAKE) == -7
    assert ex(sw=True, M=24) == -3                         # I % 16
    assert ex(flags=2) == -1 and ex(flags=-1) == -1       # unknown flag bits


def test_mx_validation_codes():
    L = qg.load(False)

    def mx(**kw):
        a = dict(fmt=6, wq=FAKE, ws=FAKE, xq=FAKE, xs=FAKE, res=None, y=FAKE, M=64, K=128, N=1)
        a.update(kw)
        return L.qgemv_mx(a["fmt"], a["wq"], a["ws"], a["xq"], a["xs"], a["res"], a["y"], a["M"], a["K"], a["N"],
                          None)
    assert mx(fmt=1) == -2 and mx(fmt=7) == -2
    assert mx(wq=None) == -1 and mx(xs=None) == -1 and mx(y=None) == -1
    assert mx(N=0) == -7 and mx(N=33) == -7
    assert mx(K=48) == -3 and mx(K=16) == -1 and mx(M=0) == -1
    assert mx(xq=ODD) == -3 and mx(wq=ODD) == -3 and mx(y=FAKE + 2) == -3
    sw = lambda **kw: L.qgemv_mx_swiglu(kw.get("fmt", 5), FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("I", 64),
                                         kw.get("K", 128), kw.get("N", 1), None)
    assert sw(fmt=3) == -2 and sw(I=0) == -1 and sw(I=24) == -3 and sw(N=33) == -7 and sw(K=40) == -3
    def swq(**kw):
        a = dict(fmt=5, hq=FAKE, hs=FAKE, I=64, K=128, N=1)
        a.update(kw)
        return L.qgemv_mx_swiglu_quant(a["fmt"], FAKE, FAKE, FAKE, FAKE, a.get("h"), a["hq"], a["hs"], a["I"], a["K"],
                                       a["N"], None)
    assert swq(fmt=3) == -2 and swq(I=0) == -1 and swq(I=48) == -3 and swq(N=33) == -7 and swq(K=40) == -3
    assert swq(hq=None) == -1 and swq(hs=None) == -1 and swq(hq=FAKE + 2) == -3 and swq(h=FAKE + 2) == -3
    # MX weights are rejected by the bf16-activation entry points
    assert _gemv(fmt=5) == -2 and _gemv(fmt=6) == -2
    aq = lambda **kw: L.qgemv_act_quant(kw.get("x", FAKE), kw.get("N", 1), kw.get("K", 64), kw.get("c", FAKE),
                                         kw.get("s", FAKE), None)
    assert aq(x=None) == -1 and aq(c=None) == -1 and aq(s=None) == -1
    assert aq(N=0) == -1 and aq(K=48) == -3 and aq(K=16) == -1
    assert aq(x=ODD) == -3 and aq(c=ODD) == -3
