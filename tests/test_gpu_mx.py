"""GPU parity of the MX path (qgemv_act_quant, qgemv_mx, qgemv_dequant for
MXFP8 / MXFP4) against the oracle, through the C ABI.

  * act_quant: codes and E8M0 scales bit for bit (one correct result);
  * dequant dump: fp32 bits equal;
  * qgemv_mx_swiglu_quant: codes and scales bit for bit against the oracle's
    quantiser of bf16(h), for the h the call also returns (that h against
    the oracle's SwiGLU at tolerance);
  * qgemv_mx: y against the oracle's GEMV of the dequantised MXFP8
    activations (quantised by the oracle, whose codes the device's equal
    bit for bit) and the dequantised weights, tolerance gemv_tolerance
    (every product is exact, only the fp32 summation rounds).
"""
import numpy as np
import pytest

import synthetic
from gpu_helpers import check_tol, dev
from oracle import dequant as D
from oracle import encodings as enc
from oracle import gemv as G
from oracle import layout as L
from oracle import quant as Q

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MX = ["mxfp8", "mxfp4"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_weight_amd as qg
    qg.load()
    yield


def qg():
    import bit_quantized_weight_amd as m
    return m


def log(*a):
    print(*a, flush=True)


def _acts(seed, N, K):
    """bf16 bits with mixed magnitudes per block, zeros, -0 and subnormals."""
    rng = synthetic.rng_for(31, seed, N, K)
    x = rng.standard_normal((N, K)).astype(np.float32)
    x *= np.exp(rng.uniform(-12, 12, (N, K // 32, 1))).repeat(32, axis=2).reshape(N, K).astype(np.float32)
    bits = synthetic.bf16_bits(x)
    if K >= 64:
        bits[0, 32:64] = 0                      # an all-zero block
    bits[:, 1] = 0x8000                         # -0
    if N > 1:
        bits[1, 2] = 0x0003                     # bf16 subnormals
        bits[1, 3] = 0x8040
    return bits


def _device_quant(xb, N, K):
    xq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((N, K // 32), dtype=torch.uint8, device="cuda")
    qg().act_quant(dev(xb, torch), xq, xs, N, K)
    torch.cuda.synchronize()
    return xq, xs


@pytest.mark.parametrize("N,K", [(1, 32), (3, 160), (16, 5120), (37, 1024)])
def test_act_quant_bit_exact(N, K):
    log("act_quant", N, K)
    xb = _acts(N * 7 + K, N, K)
    if N > 2:
        xb[2, :32] = 0x0001                     # a block of subnormals only
    xq, xs = _device_quant(xb, N, K)
    codes, e = Q.mx_act_quant(xb)
    assert np.array_equal(xs.cpu().numpy(), e), np.argwhere(xs.cpu().numpy() != e)[:5]
    got = xq.cpu().numpy()
    assert np.array_equal(got, codes), np.argwhere(got != codes)[:5]


@pytest.mark.parametrize("fmt", MX)
@pytest.mark.parametrize("M,K", [(16, 128), (37, 160), (100, 1024)])
def test_mx_dequant_dump_bit_exact(fmt, M, K):
    log("mx dequant", fmt, M, K)
    rng = synthetic.rng_for(32, M, K)
    W = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-30, 30, (M, 1)))).astype(np.float32)
    W[0, :32] = 0.0
    if M > 2:
        W[2, :32] = np.float32(2.0 ** -130)     # a clamped scale
    wq, ws = qg().pack(fmt, W)
    out = torch.full((M, K), float("nan"), dtype=torch.float32, device="cuda")
    qg().qgemv_dequant(fmt, dev(wq, torch), dev(ws, torch), M, K, out)
    torch.cuda.synchronize()
    ref = D.dequant(L.unpack(fmt, M, K, wq, ws))
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), np.argwhere(got != ref)[:5]


def _mx_case(fmt, M, K, N, seed):
    rng = synthetic.rng_for(33, seed, M, K)
    W = synthetic.weights(rng, M, K)
    wq, ws = qg().pack(fmt, W)
    xb = synthetic.activations(rng, N, K)
    return wq, ws, xb


def _run_mx(fmt, wq, ws, xb, M, K, N, residual=None, alias=False):
    xq, xs = _device_quant(xb, N, K)
    y = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda")
    r = None
    if residual is not None:
        r = dev(residual, torch)
        if alias:
            y = r
    qg().qgemv_mx(fmt, dev(wq, torch), dev(ws, torch), xq, xs, y, M, K, N, residual=r)
    torch.cuda.synchronize()
    return y.cpu().numpy(), xq, xs


def _ref(fmt, wq, ws, xb, M, K, residual=None):
    Wd = D.dequant(L.unpack(fmt, M, K, wq, ws))
    x = G.mx_activations(xb)
    return G.gemv(x, Wd, residual), G.gemv_tolerance(x, Wd)


@pytest.mark.parametrize("fmt", MX)
@pytest.mark.parametrize("M,K", [(64, 512), (37, 160), (16, 32), (300, 1024), (100, 5120), (48, 17408 // 4)])
@pytest.mark.parametrize("N", [1, 2, 5, 8, 16, 17, 32])
def test_mx_gemv_parity(fmt, M, K, N):
    log("mx gemv", fmt, M, K, N)
    wq, ws, xb = _mx_case(fmt, M, K, N, seed=N)
    y, xq, xs = _run_mx(fmt, wq, ws, xb, M, K, N)
    codes, e = Q.mx_act_quant(xb)
    assert np.array_equal(xq.cpu().numpy(), codes) and np.array_equal(xs.cpu().numpy(), e)
    ref, T = _ref(fmt, wq, ws, xb, M, K)
    check_tol(y, ref, T, f"{fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt", MX)
def test_mx_residual_aliasing_and_determinism(fmt):
    M, K, N = 200, 1024, 4
    wq, ws, xb = _mx_case(fmt, M, K, N, seed=9)
    r = synthetic.residual(np.random.default_rng(4), N, M)
    y1, _, _ = _run_mx(fmt, wq, ws, xb, M, K, N, residual=r)
    y2, _, _ = _run_mx(fmt, wq, ws, xb, M, K, N, residual=r, alias=True)
    y3, _, _ = _run_mx(fmt, wq, ws, xb, M, K, N, residual=r)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), y3.view(np.uint32))
    ref, T = _ref(fmt, wq, ws, xb, M, K, r)
    check_tol(y1, ref, T, "residual")


@pytest.mark.parametrize("fmt", MX)
@pytest.mark.parametrize("I,K,N", [(64, 512, 1), (48, 160, 3), (256, 2048, 8), (128, 1024, 16), (80, 640, 29)])
def test_mx_swiglu_parity(fmt, I, K, N):
    log("mx swiglu", fmt, I, K, N)
    wq, ws, xb = _mx_case(fmt, 2 * I, K, N, seed=I + N)
    xq, xs = _device_quant(xb, N, K)
    h = torch.full((N, I), float("nan"), dtype=torch.float32, device="cuda")
    qg().qgemv_mx_swiglu(fmt, dev(wq, torch), dev(ws, torch), xq, xs, h, I, K, N)
    torch.cuda.synchronize()
    Wd = D.dequant(L.unpack(fmt, 2 * I, K, wq, ws))
    x = G.mx_activations(xb)
    href, Th = G.swiglu_from(G.gemv(x, Wd[:I]), G.gemv(x, Wd[I:]), G.gemv_tolerance(x, Wd[:I]),
                             G.gemv_tolerance(x, Wd[I:]))
    check_tol(h.cpu().numpy(), href, Th, f"mx swiglu {fmt} I={I} K={K} N={N}")


def test_mx_swiglu_full_size_sampled_rows():
    fmt, I, K, N = "mxfp4", 17408, 5120, 4
    log("mx swiglu full", fmt, I, K, N)
    rng = synthetic.rng_for(0, 35, I, K)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, 2 * I, K))
    xb = synthetic.activations(rng, N, K, 0.01)
    xq, xs = _device_quant(xb, N, K)
    h = torch.full((N, I), float("nan"), dtype=torch.float32, device="cuda")
    qg().qgemv_mx_swiglu(fmt, dev(wq, torch), dev(ws, torch), xq, xs, h, I, K, N)
    torch.cuda.synchronize()
    hg = h.cpu().numpy()
    x = G.mx_activations(xb)
    q = L.unpack(fmt, 2 * I, K, wq, ws)
    RT = I // 16
    for rt in sorted({0, RT // 2, RT - 1, *np.random.default_rng(5).integers(0, RT, 3).tolist()}):
        def rows(t):
            sl = slice(t * 16, (t + 1) * 16)
            return D.dequant(Q.Quantized(fmt, 16, K, q.codes[sl], e=q.e[sl]))
        Wg, Wu = rows(rt), rows(RT + rt)
        href, Th = G.swiglu_from(G.gemv(x, Wg), G.gemv(x, Wu), G.gemv_tolerance(x, Wg), G.gemv_tolerance(x, Wu))
        check_tol(hg[:, rt * 16:(rt + 1) * 16], href, Th, f"tile {rt}")


def _swiglu_quant_case(fmt, wq, ws, xb, I, K, N, rows=None):
    """qgemv_mx_swiglu_quant's codes and scales, checked bit for bit against
    the oracle's MXFP8 quantiser applied to bf16 of the h the call returns
    (and against the device's act_quant of it), and that h against the
    oracle's SwiGLU (all rows, or the row tiles listed)."""
    xq, xs = _device_quant(xb, N, K)
    h = torch.full((N, I), float("nan"), dtype=torch.float32, device="cuda")
    hq = torch.full((N, I), 0xAA, dtype=torch.uint8, device="cuda")
    hs = torch.full((N, I // 32), 0xAA, dtype=torch.uint8, device="cuda")
    qg().qgemv_mx_swiglu_quant(fmt, dev(wq, torch), dev(ws, torch), xq, xs, hq, hs, I, K, N, h=h)
    torch.cuda.synchronize()
    hg = h.cpu().numpy()
    hb = synthetic.bf16_bits(hg)
    codes, e = Q.mx_act_quant(hb)
    got_c, got_e = hq.cpu().numpy(), hs.cpu().numpy()
    assert np.array_equal(got_e, e), np.argwhere(got_e != e)[:5]
    assert np.array_equal(got_c, codes), np.argwhere(got_c != codes)[:5]
    dq, ds = _device_quant(hb, N, I)
    assert np.array_equal(dq.cpu().numpy(), got_c) and np.array_equal(ds.cpu().numpy(), got_e)
    # without h the codes are the same
    hq2 = torch.zeros((N, I), dtype=torch.uint8, device="cuda")
    hs2 = torch.zeros((N, I // 32), dtype=torch.uint8, device="cuda")
    qg().qgemv_mx_swiglu_quant(fmt, dev(wq, torch), dev(ws, torch), xq, xs, hq2, hs2, I, K, N)
    torch.cuda.synchronize()
    assert np.array_equal(hq2.cpu().numpy(), got_c) and np.array_equal(hs2.cpu().numpy(), got_e)
    x = G.mx_activations(xb)
    q = L.unpack(fmt, 2 * I, K, wq, ws)
    RT = I // 16
    for rt in (range(RT) if rows is None else rows):
        def tile(t):
            sl = slice(t * 16, (t + 1) * 16)
            return D.dequant(Q.Quantized(fmt, 16, K, q.codes[sl], e=q.e[sl]))
        Wg, Wu = tile(rt), tile(RT + rt)
        href, Th = G.swiglu_from(G.gemv(x, Wg), G.gemv(x, Wu), G.gemv_tolerance(x, Wg), G.gemv_tolerance(x, Wu))
        check_tol(hg[:, rt * 16:(rt + 1) * 16], href, Th, f"h tile {rt}")
    return hb


@pytest.mark.parametrize("fmt", MX)
@pytest.mark.parametrize("I,K,N", [(32, 128, 1), (64, 512, 1), (96, 160, 3), (256, 2048, 8), (128, 1024, 16),
                                   (160, 640, 29), (64, 256, 32)])
def test_mx_swiglu_quant_bit_exact(fmt, I, K, N):
    log("mx swiglu quant", fmt, I, K, N)
    wq, ws, xb = _mx_case(fmt, 2 * I, K, N, seed=3 * I + N)
    _swiglu_quant_case(fmt, wq, ws, xb, I, K, N)


@pytest.mark.parametrize("fmt,N", [("mxfp4", 1), ("mxfp8", 8)])
def test_mx_swiglu_quant_full_size(fmt, N):
    I, K = 17408, 5120
    log("mx swiglu quant full", fmt, I, K, N)
    rng = synthetic.rng_for(0, 36, I, K)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, 2 * I, K))
    xb = synthetic.activations(rng, N, K, 0.01)
    RT = I // 16
    rows = sorted({0, 1, RT // 2, RT - 1, *np.random.default_rng(6).integers(0, RT, 3).tolist()})
    hb = _swiglu_quant_case(fmt, wq, ws, xb, I, K, N, rows=rows)
    assert np.count_nonzero(hb & 0x7FFF) > 0.99 * hb.size   # a live h, not zeros


@pytest.mark.parametrize("fmt,M,K,N", [("mxfp8", 17408, 5120, 1), ("mxfp4", 17408, 5120, 8),
                                       ("mxfp8", 5120, 17408, 16), ("mxfp4", 7168, 5120, 16),
                                       ("mxfp8", 17408, 5120, 32)])
def test_mx_full_size_sampled_rows(fmt, M, K, N):
    log("mx full", fmt, M, K, N)
    rng = synthetic.rng_for(0, 34, M, K)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, M, K))
    xb = synthetic.activations(rng, N, K, 0.01)
    y, _, _ = _run_mx(fmt, wq, ws, xb, M, K, N)
    x = G.mx_activations(xb)
    RT = M // 16
    q = L.unpack(fmt, M, K, wq, ws)
    for rt in sorted({0, 1, RT // 2, RT - 1, *np.random.default_rng(3).integers(0, RT, 4).tolist()}):
        rows = slice(rt * 16, (rt + 1) * 16)
        sub = Q.Quantized(fmt, 16, K, q.codes[rows], e=q.e[rows])
        Wt = D.dequant(sub)
        check_tol(y[:, rows], G.gemv(x, Wt), G.gemv_tolerance(x, Wt), f"tile {rt}")
