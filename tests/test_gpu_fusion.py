"""GPU parity of the fused RMSNorm prologue and bf16 output (qgemv_ex,
qgemv_swiglu_ex) against the oracle, through the C ABI.

Tolerance per output (oracle): the GEMV bound with the normalisation's own
term, (2e-3 + norm_rel(K)) * sum|x W| + 1e-5, x the fp64 RMSNorm; SwiGLU
propagated as for qgemv_swiglu. The bf16 output equals the bf16 rounding of
the same call's fp32 output bit for bit.
"""
import numpy as np
import pytest

import synthetic
from gpu_helpers import FORMATS, check_tol, dev, make_case, oracle_weights, tile_rows
from oracle import encodings as enc
from oracle import gemv as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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


def _norm_inputs(seed, N, K):
    rng = synthetic.rng_for(21, seed, N, K)
    h = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(2.5)).astype(np.float32)
    gamma = (1.0 + 0.2 * rng.standard_normal(K)).astype(np.float32)
    return h, gamma


def _bf16_of(y32):
    return synthetic.bf16_bits(np.asarray(y32, np.float32))


def _run_ex(fmt, wq, ws, h, gamma, M, K, N, eps, residual=None, swiglu=False):
    out = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda")
    obf = torch.zeros((N, M), dtype=torch.int16, device="cuda")
    args = dict(norm_src=dev(h, torch), norm_gamma=dev(gamma, torch), norm_eps=eps, out_bf16=obf)
    if swiglu:
        qg().qgemv_swiglu_ex(fmt, dev(wq, torch), dev(ws, torch), None, out, M, K, N, **args)
    else:
        qg().qgemv_ex(fmt, dev(wq, torch), dev(ws, torch), None, out, M, K, N,
                      residual=None if residual is None else dev(residual, torch), **args)
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    yb = obf.cpu().numpy().view(np.uint16)
    assert np.array_equal(yb, _bf16_of(y)), "bf16 output differs from the rounded fp32 output"
    return y, yb


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,K,N", [(64, 512, 1), (37, 160, 3), (200, 1024, 8), (48, 4096, 2), (40, 32768, 1),
                                   (48, 32768, 2), (33, 32768, 3)])
def test_norm_gemv_parity(fmt, M, K, N):
    log("norm gemv", fmt, M, K, N)
    W, _, wq, ws = make_case(fmt, M, K, N, seed=41)
    h, gamma = _norm_inputs(M, N, K)
    r = synthetic.residual(np.random.default_rng(M), N, M)
    y, yb = _run_ex(fmt, wq, ws, h, gamma, M, K, N, 1e-5, residual=r)
    Wd = oracle_weights(fmt, wq, ws, M, K)
    x = G.rmsnorm(h, gamma, 1e-5)
    ref = G.gemv(x, Wd, r)
    T = G.norm_gemv_tolerance(x, Wd)
    check_tol(y, ref, T, f"norm gemv {fmt}")
    check_tol(enc.f32_from_bf16_bits(yb), ref, T + G.BF16_REL * np.abs(ref), "bf16 output")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("I,K,N", [(64, 512, 1), (48, 160, 3), (256, 2048, 8)])
def test_norm_swiglu_parity(fmt, I, K, N):
    log("norm swiglu", fmt, I, K, N)
    W, _, wq, ws = make_case(fmt, 2 * I, K, N, seed=43)
    h, gamma = _norm_inputs(I, N, K)
    hv, hb = _run_ex(fmt, wq, ws, h, gamma, I, K, N, 1e-6, swiglu=True)
    Wd = oracle_weights(fmt, wq, ws, 2 * I, K)
    x = G.rmsnorm(h, gamma, 1e-6)
    g, u = G.gemv(x, Wd[:I]), G.gemv(x, Wd[I:])
    href, Th = G.swiglu_from(g, u, G.norm_gemv_tolerance(x, Wd[:I]), G.norm_gemv_tolerance(x, Wd[I:]))
    check_tol(hv, href, Th, f"norm swiglu {fmt}")


def test_bf16_output_without_norm_equals_plain_call():
    """The fusion struct with only a bf16 output: the fp32 result is the
    plain qgemv's, bit for bit, and the bf16 copy is its rounding."""
    M, K, N = 96, 1024, 4
    W, xb, wq, ws = make_case("int4", M, K, N, seed=45)
    y1 = torch.empty((N, M), dtype=torch.float32, device="cuda")
    qg().qgemv("int4", dev(wq, torch), dev(ws, torch), dev(xb, torch), y1, M, K, N)
    y2 = torch.empty((N, M), dtype=torch.float32, device="cuda")
    yb = torch.zeros((N, M), dtype=torch.int16, device="cuda")
    qg().qgemv_ex("int4", dev(wq, torch), dev(ws, torch), dev(xb, torch), y2, M, K, N, out_bf16=yb)
    yo = torch.zeros((N, M), dtype=torch.int16, device="cuda")
    qg().qgemv_ex("int4", dev(wq, torch), dev(ws, torch), dev(xb, torch), None, M, K, N, out_bf16=yo)
    torch.cuda.synchronize()
    a, b = y1.cpu().numpy(), y2.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(yb.cpu().numpy().view(np.uint16), _bf16_of(a))
    assert np.array_equal(yo.cpu().numpy().view(np.uint16), _bf16_of(a))


@pytest.mark.parametrize("fmt,M,K,N,sw", [("int5", 2 * 17408, 5120, 1, True), ("int5", 2 * 17408, 5120, 8, True),
                                          ("int5", 5120, 17408, 8, False), ("nvfp4", 7168, 5120, 4, False),
                                          ("int4", 17408, 5120, 1, False), ("int4", 2 * 17408, 5120, 2, True),
                                          ("int5", 2 * 17408, 5120, 4, True), ("nvfp4", 2 * 17408, 5120, 3, True)])
def test_norm_full_size_sampled_rows(fmt, M, K, N, sw):
    """Full-size shapes (both activation staging paths: whole range in LDS,
    and the ring; gate/up pairs with whole-K waves at 1-2 tokens and the ring
    at 3-4); the oracle recomputes sampled row tiles."""
    log("norm full", fmt, M, K, N, sw)
    rng = synthetic.rng_for(0, 8, M, K)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, M, K))
    h, gamma = _norm_inputs(K, N, K)
    Mo = M // 2 if sw else M
    y, _ = _run_ex(fmt, wq, ws, h, gamma, Mo, K, N, 1e-6, swiglu=sw)
    x = G.rmsnorm(h, gamma, 1e-6)
    RT = Mo // 16
    for rt in sorted({0, RT // 2, RT - 1, *np.random.default_rng(2).integers(0, RT, 3).tolist()}):
        if sw:
            Wg = tile_rows(fmt, wq, ws, M, K, rt)
            Wu = tile_rows(fmt, wq, ws, M, K, RT + rt)
            href, Th = G.swiglu_from(G.gemv(x, Wg), G.gemv(x, Wu), G.norm_gemv_tolerance(x, Wg),
                                     G.norm_gemv_tolerance(x, Wu))
            check_tol(y[:, rt * 16:(rt + 1) * 16], href, Th, f"tile {rt}")
        else:
            Wt = tile_rows(fmt, wq, ws, M, K, rt)
            check_tol(y[:, rt * 16:(rt + 1) * 16], G.gemv(x, Wt), G.norm_gemv_tolerance(x, Wt), f"tile {rt}")


def test_chained_mlp_block():
    """One MLP block chained on the device: RMSNorm(residual) -> gate/up +
    SwiGLU with a bf16 h -> down projection of that bf16 h + residual. The
    oracle runs the same chain in fp64 from the same inputs; its bound carries
    the SwiGLU bound and one bf16 rounding of h through the down projection."""
    I, H, N = 256, 1024, 3
    rng = synthetic.rng_for(22, I, H)
    wgu, sgu = qg().pack("int5", synthetic.weights(rng, 2 * I, H))
    wdn, sdn = qg().pack("int5", synthetic.weights(rng, H, I))
    res, gamma = _norm_inputs(5, N, H)
    hbuf = torch.zeros((N, I), dtype=torch.int16, device="cuda")
    y = torch.empty((N, H), dtype=torch.float32, device="cuda")
    dres = dev(res, torch)
    qg().qgemv_swiglu_ex("int5", dev(wgu, torch), dev(sgu, torch), None, None, I, H, N, norm_src=dres,
                         norm_gamma=dev(gamma, torch), norm_eps=1e-6, out_bf16=hbuf)
    qg().qgemv("int5", dev(wdn, torch), dev(sdn, torch), hbuf, y, H, I, N, residual=dres)
    torch.cuda.synchronize()
    Wgu = oracle_weights("int5", wgu, sgu, 2 * I, H)
    Wdn = oracle_weights("int5", wdn, sdn, H, I).astype(np.float64)
    x = G.rmsnorm(res, gamma, 1e-6)
    href, Th = G.swiglu_from(G.gemv(x, Wgu[:I]), G.gemv(x, Wgu[I:]), G.norm_gemv_tolerance(x, Wgu[:I]),
                             G.norm_gemv_tolerance(x, Wgu[I:]))
    y_ref = G.gemv(href, Wdn, res)
    T = G.chain_tolerance(href, Th, Wdn)                  # h crosses the chain as bf16
    check_tol(y.cpu().numpy(), y_ref, T, "chained MLP block")


def test_chained_mlp_block_in_a_hip_graph():
    """The chained MLP block (two launches, no allocation, no synchronisation)
    captured in a HIP graph and replayed several times, with other eager GPU
    work and synchronisations between the replays: every replay equals the
    eager result bit for bit."""
    I, H, N = 512, 2048, 2
    rng = synthetic.rng_for(23, I, H)
    wgu, sgu = (dev(a, torch) for a in qg().pack("int4", synthetic.weights(rng, 2 * I, H)))
    wdn, sdn = (dev(a, torch) for a in qg().pack("int5", synthetic.weights(rng, H, I)))
    res, gamma = _norm_inputs(6, N, H)
    dres, dg = dev(res, torch), dev(gamma, torch)
    hbuf = torch.zeros((N, I), dtype=torch.int16, device="cuda")
    y = torch.zeros((N, H), dtype=torch.float32, device="cuda")

    def chain():
        qg().qgemv_swiglu_ex("int4", wgu, sgu, None, None, I, H, N, norm_src=dres, norm_gamma=dg, norm_eps=1e-6,
                             out_bf16=hbuf)
        qg().qgemv("int5", wdn, sdn, hbuf, y, H, I, N, residual=dres)

    chain()
    torch.cuda.synchronize()
    eager = y.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    noise = torch.randn((N, H), device="cuda")
    for rep in range(4):
        y.fill_(float("nan"))
        hbuf.zero_()
        _ = (noise * rep).sum()                 # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"replay {rep} differs"


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,K,swiglu,norm", [(128, 1024, False, False), (37, 5120, False, True),
                                             (64, 2048, True, False), (48, 640, True, True),
                                             (17408, 5120, False, False)])
def test_batch_invariant_mode(fmt, M, K, swiglu, norm):
    """QGEMV_BATCH_INVARIANT: each token of an N = 8 call, of an N = 3 call on
    rows 5..7 and of N = 1 calls gives the same bits, and all stay within the
    oracle's bound."""
    log("batch invariant", fmt, M, K, swiglu, norm)
    Mp = 2 * M if swiglu else M
    rng = synthetic.rng_for(24, M, K)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, Mp, K))
    dq, dsc = dev(wq, torch), dev(ws, torch)
    if norm:
        h, gamma = _norm_inputs(M + K, 8, K)
        dg = dev(gamma, torch)
    else:
        xb = synthetic.activations(rng, 8, K, 0.01)

    def call(rows):
        n = len(rows)
        out = torch.full((n, M), float("nan"), dtype=torch.float32, device="cuda")
        kw = dict(batch_invariant=True)
        if norm:
            kw.update(norm_src=dev(np.ascontiguousarray(h[rows]), torch), norm_gamma=dg, norm_eps=1e-6)
            x = None
        else:
            x = dev(np.ascontiguousarray(xb[rows]), torch)
        if swiglu:
            qg().qgemv_swiglu_ex(fmt, dq, dsc, x, out, M, K, n, **kw)
        else:
            qg().qgemv_ex(fmt, dq, dsc, x, out, M, K, n, **kw)
        torch.cuda.synchronize()
        return out.cpu().numpy()
    y8 = call(list(range(8)))
    y3 = call([5, 6, 7])
    for n in range(8):
        y1 = call([n])
        assert np.array_equal(y1.view(np.uint32)[0], y8.view(np.uint32)[n]), f"row {n}: N=1 differs from N=8"
    assert np.array_equal(y3.view(np.uint32), y8.view(np.uint32)[5:8]), "N=3 differs from N=8"
    if M > 1024:                                   # full size: check sampled tiles against the oracle
        x64 = G.x_from_bits(xb)
        for rt in (0, 511, 1087):
            Wt = tile_rows(fmt, wq, ws, M, K, rt)
            check_tol(y8[:, rt * 16:(rt + 1) * 16], G.gemv(x64, Wt), G.gemv_tolerance(x64, Wt), f"tile {rt}")
        return
    Wd = oracle_weights(fmt, wq, ws, Mp, K)
    x64 = G.rmsnorm(h, gamma, 1e-6) if norm else G.x_from_bits(xb)
    tol = G.norm_gemv_tolerance if norm else G.gemv_tolerance
    if swiglu:
        ref, T = G.swiglu_from(G.gemv(x64, Wd[:M]), G.gemv(x64, Wd[M:]), tol(x64, Wd[:M]), tol(x64, Wd[M:]))
    else:
        ref, T = G.gemv(x64, Wd), tol(x64, Wd)
    check_tol(y8, ref, T, "batch invariant")
