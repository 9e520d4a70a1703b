"""GPU parity of the split-remainder launch (qgemv_ex / qgemv_swiglu_ex with a
workspace) against the oracle, through the C ABI.

The leftover row blocks of these shapes are cut into K fragments whose
partial sums meet in the workspace; the oracle recomputes sampled row tiles,
most of them from the split blocks at the end of the matrix. Tolerance as for
qgemv (oracle gemv_tolerance; SwiGLU propagated by swiglu_from). The split
changes the summation order only, so the same call repeated gives the same
bits, and the workspace's flags are back at zero after every call.
"""
import numpy as np
import pytest

import synthetic
from gpu_helpers import check_tol, dev, tile_rows
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


def _flag_bytes():
    # sticky word and padding (256 bytes), then one 64-byte flag per partial slot (7 per compute unit)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return 256 + 64 * 7 * cus


def _call(fmt, wq, ws, xb, Mo, K, N, sw, wsp=None, residual=None, out_bf16=None):
    y = torch.full((N, Mo), float("nan"), dtype=torch.float32, device="cuda")
    if sw:
        qg().qgemv_swiglu_ex(fmt, wq, ws, xb, y, Mo, K, N, workspace=wsp, out_bf16=out_bf16)
    else:
        qg().qgemv_ex(fmt, wq, ws, xb, y, Mo, K, N, residual=residual, workspace=wsp, out_bf16=out_bf16)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _sample_tiles(RT, seed):
    # the split blocks sit at the end: take the last tiles densely
    tail = list(range(max(0, RT - 6), RT))
    rnd = np.random.default_rng(seed).integers(max(0, RT - RT // 4), RT, 4).tolist()
    return sorted({0, RT // 2, *tail, *rnd})


# Shapes whose row blocks leave a remainder on 256 compute units (taken:
# the split is expected on MI355X, so its bits must differ somewhere from the
# unsplit call's):
#   gate/up pairs [2 x 17408][5120]: 1088 blocks = 1024 + 64 (4 fragments)
#   [17408][5120] one tile per workgroup: 1088 blocks (4 fragments)
#   [5120][17408] one tile per workgroup (NVFP4 and int8 at N = 2): 320 blocks = 256 + 64
# and shapes where it is declined (grid not resident at once, or a remainder
# above half the units), which must still be right.
SHAPES = [("int5", 2 * 17408, 5120, 1, True, True), ("nvfp4", 2 * 17408, 5120, 1, True, True),
          ("int4", 2 * 17408, 5120, 8, True, True), ("int8", 2 * 17408, 5120, 8, True, True),
          ("int4", 17408, 5120, 1, False, True), ("int8", 17408, 5120, 8, False, True),
          ("nvfp4", 5120, 17408, 2, False, True), ("int8", 5120, 17408, 2, False, True),
          ("int4", 2 * 17408, 5120, 2, True, False), ("int4", 7168, 5120, 2, False, False),
          # gate/up pairs at 5-8 tokens read their activations by direct loads
          ("int5", 2 * 17408, 5120, 5, True, True), ("nvfp4", 2 * 17408, 5120, 6, True, True)]


@pytest.mark.parametrize("fmt,M,K,N,sw,taken", SHAPES)
def test_split_full_size_sampled_tiles(fmt, M, K, N, sw, taken):
    log("split", fmt, M, K, N, sw)
    rng = synthetic.rng_for(0, 11, M, K)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, M, K))
    xb = synthetic.activations(rng, N, K)
    Mo = M // 2 if sw else M
    r = None if sw else synthetic.residual(np.random.default_rng(M), N, Mo)
    wqd, wsd, xd = dev(wq, torch), dev(ws, torch), dev(xb, torch)
    rd = None if r is None else dev(r, torch)
    wsp = qg().split_workspace(torch.device("cuda:0"))
    obf = torch.zeros((N, Mo), dtype=torch.int16, device="cuda")
    y = _call(fmt, wqd, wsd, xd, Mo, K, N, sw, wsp, rd, out_bf16=obf)
    w = wsp.cpu().numpy()
    assert not w[:_flag_bytes()].any(), "flags or the error word not zero after the call"
    assert np.array_equal(obf.cpu().numpy().view(np.uint16), synthetic.bf16_bits(y)), "bf16 output"
    y2 = _call(fmt, wqd, wsd, xd, Mo, K, N, sw, wsp, rd)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "split result not reproducible"
    y0 = _call(fmt, wqd, wsd, xd, Mo, K, N, sw, None, rd)       # the unsplit launch
    if taken:
        assert not np.array_equal(y.view(np.uint32), y0.view(np.uint32)), "split not taken"
    x = G.x_from_bits(xb)
    RT = Mo // 16
    for rt in _sample_tiles(RT, M + N):
        cols = slice(rt * 16, (rt + 1) * 16)
        if sw:
            Wg = tile_rows(fmt, wq, ws, M, K, rt)
            Wu = tile_rows(fmt, wq, ws, M, K, RT + rt)
            ref, T = G.swiglu_from(G.gemv(x, Wg), G.gemv(x, Wu), G.gemv_tolerance(x, Wg), G.gemv_tolerance(x, Wu))
        else:
            Wt = tile_rows(fmt, wq, ws, M, K, rt)
            ref, T = G.gemv(x, Wt, r[:, cols]), G.gemv_tolerance(x, Wt)
        check_tol(y[:, cols], ref, T, f"split tile {rt}")
        check_tol(y0[:, cols], ref, T, f"unsplit tile {rt}")


def test_split_workspace_reuse_across_shapes():
    """One workspace, calls of different shapes and N in stream order: each
    result equals that of the same call on a fresh workspace."""
    fmt, K = "int4", 5120
    rng = synthetic.rng_for(0, 12, K)
    W = synthetic.weights(rng, 2 * 17408, K)
    wq, ws = qg().pack(fmt, W)
    wq2, ws2 = qg().pack(fmt, W[:7168])
    wsp = qg().split_workspace(torch.device("cuda:0"))
    cases = [(wq, ws, 17408, 1, True), (wq2, ws2, 7168, 2, False), (wq, ws, 17408, 8, True), (wq, ws, 17408, 1, True)]
    for i, (a, b, Mo, N, sw) in enumerate(cases):
        log("reuse", i, Mo, N, sw)
        xd = dev(synthetic.activations(rng, N, K), torch)
        ad, bd = dev(a, torch), dev(b, torch)
        y = _call(fmt, ad, bd, xd, Mo, K, N, sw, wsp)
        yf = _call(fmt, ad, bd, xd, Mo, K, N, sw, qg().split_workspace(torch.device("cuda:0")))
        assert np.array_equal(y.view(np.uint32), yf.view(np.uint32)), f"case {i}"
    assert not wsp.cpu().numpy()[:_flag_bytes()].any()


def test_split_workspace_errors():
    fmt, M, K, N = "int4", 256, 512, 1
    rng = synthetic.rng_for(0, 13, M, K)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, M, K))
    wqd, wsd = dev(wq, torch), dev(ws, torch)
    xd = dev(synthetic.activations(rng, N, K), torch)
    y = torch.empty((N, M), dtype=torch.float32, device="cuda")
    n = qg().split_workspace_bytes()
    assert n > _flag_bytes()
    small = torch.zeros(n - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(qg().QgemvError) as e:
        qg().qgemv_ex(fmt, wqd, wsd, xd, y, M, K, N, workspace=small)
    assert e.value.status == -5   # QGEMV_EWORKSPACE
    big = torch.zeros(n + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(qg().QgemvError) as e:
        qg().qgemv_ex(fmt, wqd, wsd, xd, y, M, K, N, workspace=big[16:16 + n])
    assert e.value.status == -3   # QGEMV_EALIGN
    # a shape with nothing to balance runs unsplit and matches the call without a workspace
    qg().qgemv_ex(fmt, wqd, wsd, xd, y, M, K, N, workspace=big[:n])
    y1 = y.clone()
    qg().qgemv_ex(fmt, wqd, wsd, xd, y, M, K, N)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y.view(torch.int32))


def test_split_and_mx_calls_in_a_hip_graph():
    """Split-remainder calls (whose fragments hand partial sums over through
    flags that every call clears itself) and an MX quantise + GEMV pair,
    captured in one HIP graph and replayed with eager work in between: every
    replay equals the eager result bit for bit, and the workspace's flags are
    back at zero."""
    K, I, N = 5120, 17408, 1
    rng = synthetic.rng_for(0, 14, K)
    W = synthetic.weights(rng, 2 * I, K)
    wq, ws = (dev(a, torch) for a in qg().pack("int5", W))
    mq, ms = (dev(a, torch) for a in qg().pack("mxfp4", W[:I]))
    x = dev(synthetic.activations(rng, N, K), torch)
    wsp = qg().split_workspace(torch.device("cuda:0"))
    h = torch.zeros((N, I), dtype=torch.float32, device="cuda")
    y = torch.zeros((N, I), dtype=torch.float32, device="cuda")
    xq = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    xs = torch.zeros((N, K // 32), dtype=torch.uint8, device="cuda")

    def calls():
        qg().qgemv_swiglu_ex("int5", wq, ws, x, h, I, K, N, workspace=wsp)
        qg().act_quant(x, xq, xs, N, K)
        qg().qgemv_mx("mxfp4", mq, ms, xq, xs, y, I, K, N)

    calls()
    torch.cuda.synchronize()
    eh, ey = h.cpu().numpy().copy(), y.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    noise = torch.randn((64, 1024), device="cuda")
    for rep in range(4):
        h.fill_(float("nan"))
        y.fill_(float("nan"))
        xq.zero_()
        _ = (noise * rep).sum()                 # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(h.cpu().numpy().view(np.uint32), eh.view(np.uint32)), f"replay {rep}: split SwiGLU"
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ey.view(np.uint32)), f"replay {rep}: MX GEMV"
        assert not wsp.cpu().numpy()[:_flag_bytes()].any(), f"replay {rep}: flags left set"


# RMSNorm prologue with the split: the fragments also publish their parts of
# each token's sum of squares (gate/up pairs at N = 1 and 8: 1024 + 64 x 4;
# [17408][5120] one tile per workgroup: 1088 = 1024 + 64 x 4). At N = 4 the
# NVFP4 prologue kernel's three-wave workgroups of the split grid (1280) do
# not all fit the chip at once, so the split is declined there.
NORM_SHAPES = [("int5", 2 * 17408, 5120, 1, True, True), ("int4", 2 * 17408, 5120, 8, True, True),
               ("nvfp4", 17408, 5120, 4, False, False), ("int8", 17408, 5120, 1, False, True)]


@pytest.mark.parametrize("fmt,M,K,N,sw,taken", NORM_SHAPES)
def test_split_with_rmsnorm_prologue(fmt, M, K, N, sw, taken):
    log("split norm", fmt, M, K, N, sw)
    rng = synthetic.rng_for(0, 13, M, K)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, M, K))
    h = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(2.5)).astype(np.float32)
    gamma = (1.0 + 0.2 * rng.standard_normal(K)).astype(np.float32)
    Mo = M // 2 if sw else M
    wqd, wsd, hd, gd = dev(wq, torch), dev(ws, torch), dev(h, torch), dev(gamma, torch)
    wsp = qg().split_workspace(torch.device("cuda:0"))

    def call(workspace):
        y = torch.full((N, Mo), float("nan"), dtype=torch.float32, device="cuda")
        f = qg().qgemv_swiglu_ex if sw else qg().qgemv_ex
        f(fmt, wqd, wsd, None, y, Mo, K, N, norm_src=hd, norm_gamma=gd, norm_eps=1e-6, workspace=workspace)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    y = call(wsp)
    assert not wsp.cpu().numpy()[:_flag_bytes()].any(), "flags or the error word not zero after the call"
    y2 = call(wsp)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "split result not reproducible"
    y0 = call(None)
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32)) != taken, "split taken" if not taken else "not taken"
    x = G.rmsnorm(h, gamma, 1e-6)
    RT = Mo // 16
    for rt in _sample_tiles(RT, M + N):
        cols = slice(rt * 16, (rt + 1) * 16)
        if sw:
            Wg = tile_rows(fmt, wq, ws, M, K, rt)
            Wu = tile_rows(fmt, wq, ws, M, K, RT + rt)
            ref, T = G.swiglu_from(G.gemv(x, Wg), G.gemv(x, Wu), G.norm_gemv_tolerance(x, Wg),
                                   G.norm_gemv_tolerance(x, Wu))
        else:
            Wt = tile_rows(fmt, wq, ws, M, K, rt)
            ref, T = G.gemv(x, Wt), G.norm_gemv_tolerance(x, Wt)
        check_tol(y[:, cols], ref, T, f"split norm tile {rt}")
        check_tol(y0[:, cols], ref, T, f"unsplit norm tile {rt}")
