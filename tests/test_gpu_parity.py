"""GPU parity of the HIP path against the oracle, through the C ABI.

Bit-exact: the dequantised-weight dump and the MoE routing index.
Tolerance (per output, from the oracle): |y - y_ref| <= 2e-3 sum|x w| + 1e-5,
SwiGLU and MoE bounds propagated as stated in oracle/gemv.py.
"""
import numpy as np
import pytest

import synthetic
from gpu_helpers import FORMATS, check_tol, dev, make_case, moe_case, oracle_weights, ref_gemv, tile_rows
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


# ------------------------------------------------------------- dequant dump

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,K", [(16, 128), (1, 32), (37, 160), (64, 1024), (100, 5120)])
def test_dequant_dump_bit_exact(fmt, M, K):
    log("dump", fmt, M, K)
    W, _, wq, ws = make_case(fmt, M, K, 1, seed=1)
    out = torch.empty((M, K), dtype=torch.float32, device="cuda")
    qg().qgemv_dequant(fmt, dev(wq, torch), dev(ws, torch), M, K, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle_weights(fmt, wq, ws, M, K)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
        np.argwhere(got.view(np.uint32) != ref.view(np.uint32))[:5]


@pytest.mark.parametrize("fmt", FORMATS)
def test_dequant_dump_all_codes_and_scales(fmt):
    """Every code value under scale fields spanning the encodings (fp16
    subnormal/normal/large, every finite E4M3 byte), compared bit for bit."""
    rng = np.random.default_rng(3)
    M, K = 48, 512
    if fmt == "int8":
        codes = rng.integers(-128, 128, (M, K)).astype(np.int8)
    else:
        codes = rng.integers(0, 32 if fmt == "int5" else 16, (M, K)).astype(np.uint8)
    if fmt == "nvfp4":
        fin = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
        sb = rng.choice(fin, (M, K // 16)).astype(np.uint8)
        wq, ws = qg().pack_codes(fmt, codes, sb, None, 0.0123)
    else:
        f16 = np.array([b for b in range(0, 0x7C00, 7)] + [b | 0x8000 for b in range(0, 0x7C00, 11)], np.uint16)
        d = rng.choice(f16, (M, K // 32)).astype(np.uint16)
        m = None if fmt == "int8" else rng.choice(f16, (M, K // 32)).astype(np.uint16)
        wq, ws = qg().pack_codes(fmt, codes, d, m)
    out = torch.empty((M, K), dtype=torch.float32, device="cuda")
    qg().qgemv_dequant(fmt, dev(wq, torch), dev(ws, torch), M, K, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle_weights(fmt, wq, ws, M, K)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), np.argwhere(~same)[:5]


# ------------------------------------------------------------------- GEMV

# (48, 32768): K long enough that every N stages its activations through the
# four-record LDS ring (N < 4 leaves lanes past the record)
SHAPES = [(1024, 1024), (37, 160), (16, 32), (100, 5120), (64, 17408 // 4), (48, 32768)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 12, 16, 20, 32])
def test_qgemv_parity(fmt, M, K, N):
    log("gemv", fmt, M, K, N)
    W, xb, wq, ws = make_case(fmt, M, K, N, seed=N)
    y = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda")
    yr, T = ref_gemv(fmt, wq, ws, xb, M, K)
    qg().qgemv(fmt, dev(wq, torch), dev(ws, torch), dev(xb, torch), y, M, K, N)
    torch.cuda.synchronize()
    check_tol(y.cpu().numpy(), yr, T, f"{fmt} M={M} K={K} N={N}")


def test_config1_int4_1024():
    """The single-GEMV workload: M = K = 1024, int4, N = 1, seed 0."""
    rng = np.random.default_rng(0)
    W = synthetic.weights(rng, 1024, 1024)
    xb = synthetic.activations(rng, 1, 1024)
    wq, ws = qg().pack("int4", W)
    yr, T = ref_gemv("int4", wq, ws, xb, 1024, 1024)
    y = torch.empty((1, 1024), dtype=torch.float32, device="cuda")
    qg().qgemv("int4", dev(wq, torch), dev(ws, torch), dev(xb, torch), y, 1024, 1024, 1)
    torch.cuda.synchronize()
    check_tol(y.cpu().numpy(), yr, T, "config1")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N", [3, 12, 27])
def test_residual_and_aliasing(fmt, N):
    M, K = 96, 640
    log("residual", fmt, N)
    W, xb, wq, ws = make_case(fmt, M, K, N, seed=11)
    r = synthetic.residual(np.random.default_rng(4), N, M)
    yr, T = ref_gemv(fmt, wq, ws, xb, M, K, residual=r)
    y = torch.empty((N, M), dtype=torch.float32, device="cuda")
    args = (dev(wq, torch), dev(ws, torch), dev(xb, torch))
    qg().qgemv(fmt, *args, y, M, K, N, residual=dev(r, torch))
    yy = dev(r, torch)                       # y aliases the residual
    qg().qgemv(fmt, *args, yy, M, K, N, residual=yy)
    torch.cuda.synchronize()
    check_tol(y.cpu().numpy(), yr, T, "residual")
    assert np.array_equal(yy.cpu().numpy(), y.cpu().numpy())


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N", [8, 20])
def test_determinism_and_canaries(fmt, N):
    M, K = 200, 2048
    log("canaries", fmt, N)
    W, xb, wq, ws = make_case(fmt, M, K, N, seed=12)
    pad = 64
    buf = torch.full((N * M + 2 * pad,), 12345.0, dtype=torch.float32, device="cuda")
    y = buf[pad: pad + N * M]
    args = (dev(wq, torch), dev(ws, torch), dev(xb, torch))
    qg().qgemv(fmt, *args, y, M, K, N)
    torch.cuda.synchronize()
    first = y.cpu().numpy().copy()
    qg().qgemv(fmt, *args, y, M, K, N)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:pad] == 12345.0) and np.all(b[pad + N * M:] == 12345.0)
    assert np.array_equal(first.view(np.uint32), y.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("fmt", FORMATS)
def test_special_cases(fmt):
    M, K = 48, 256
    # zero weights: y == residual exactly
    zero = np.zeros((M, K), np.float32)
    wq, ws = qg().pack(fmt, zero)
    xb = synthetic.activations(np.random.default_rng(1), 2, K)
    r = synthetic.residual(np.random.default_rng(2), 2, M)
    y = torch.empty((2, M), dtype=torch.float32, device="cuda")
    qg().qgemv(fmt, dev(wq, torch), dev(ws, torch), dev(xb, torch), y, M, K, 2, residual=dev(r, torch))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), r)
    # one-hot x picks one column of the dequantised matrix
    W, _, wq, ws = make_case(fmt, M, K, 1, seed=5)
    Wd = oracle_weights(fmt, wq, ws, M, K)
    for k in (0, 77, 255):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        xb = synthetic.bf16_bits(x)
        y1 = torch.empty((1, M), dtype=torch.float32, device="cuda")
        qg().qgemv(fmt, dev(wq, torch), dev(ws, torch), dev(xb, torch), y1, M, K, 1)
        torch.cuda.synchronize()
        T = G.gemv_tolerance(x.astype(np.float64), Wd)
        check_tol(y1.cpu().numpy(), Wd[:, k][None, :].astype(np.float64), T, f"one-hot k={k}")
    # 16 one-hot tokens in one call (one operand slot): token t picks column ks[t]
    ks = np.random.default_rng(6).choice(K, 16, replace=False)
    x = np.zeros((16, K), np.float32)
    x[np.arange(16), ks] = 1.0
    y16 = torch.empty((16, M), dtype=torch.float32, device="cuda")
    qg().qgemv(fmt, dev(wq, torch), dev(ws, torch), dev(synthetic.bf16_bits(x), torch), y16, M, K, 16)
    torch.cuda.synchronize()
    check_tol(y16.cpu().numpy(), Wd[:, ks].T.astype(np.float64), G.gemv_tolerance(x.astype(np.float64), Wd),
              "one-hot batch of 16")


@pytest.mark.parametrize("fmt", FORMATS)
def test_batch_invariance(fmt):
    """Row n of an N = 8 call agrees with an N = 1 call on x[n] (tolerance;
    the bitwise-equal fraction is printed)."""
    M, K = 128, 1024
    W, xb, wq, ws = make_case(fmt, M, K, 8, seed=21)
    args = (dev(wq, torch), dev(ws, torch))
    y8 = torch.empty((8, M), dtype=torch.float32, device="cuda")
    qg().qgemv(fmt, *args, dev(xb, torch), y8, M, K, 8)
    yr, T = ref_gemv(fmt, wq, ws, xb, M, K)
    eq = 0
    for n in range(8):
        y1 = torch.empty((1, M), dtype=torch.float32, device="cuda")
        qg().qgemv(fmt, *args, dev(xb[n:n + 1], torch), y1, M, K, 1)
        torch.cuda.synchronize()
        a, b = y1.cpu().numpy()[0], y8.cpu().numpy()[n]
        check_tol(a[None], yr[n:n + 1], T[n:n + 1], "N=1")
        eq += int(np.sum(a.view(np.uint32) == b.view(np.uint32)))
    log(f"batch invariance {fmt}: bitwise equal fraction {eq / (8 * M):.3f}")


# ----------------------------------------------------------------- SwiGLU

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("I,K,N", [(64, 512, 1), (48, 160, 3), (256, 2048, 8), (768, 2048, 4), (96, 1024, 16),
                                   (32, 32768, 11), (80, 640, 27), (64, 5120, 32)])
def test_swiglu_parity(fmt, I, K, N):
    log("swiglu", fmt, I, K, N)
    W, xb, wq, ws = make_case(fmt, 2 * I, K, N, seed=31)
    Wd = oracle_weights(fmt, wq, ws, 2 * I, K)
    x = G.x_from_bits(xb)
    h_ref, Th = G.swiglu(x, Wd)
    h = torch.full((N, I), float("nan"), dtype=torch.float32, device="cuda")
    qg().qgemv_swiglu(fmt, dev(wq, torch), dev(ws, torch), dev(xb, torch), h, I, K, N)
    torch.cuda.synchronize()
    check_tol(h.cpu().numpy(), h_ref, Th, f"swiglu {fmt}")


# -------------------------------------------------------------------- MoE

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N", [1, 3, 8])
def test_moe_parity(fmt, N):
    E, H, I, k = 16, 256, 64, 4
    log("moe", fmt, N)
    bufs, Wgu, Wdn, xb, ids, gates, r = moe_case(fmt, E, H, I, N, k, seed=N)
    y_ref, T = G.moe(G.x_from_bits(xb), ids, gates, Wgu, Wdn, r)
    nbytes = qg().moe_workspace_bytes(E, H, I, N, k)
    wsp = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((N, H), dtype=torch.float32, device="cuda")
    d = [dev(b, torch) for b in bufs]
    qg().qgemv_moe(fmt, *d, E, H, I, dev(xb, torch), dev(ids, torch), dev(gates, torch), k, y, N, wsp, nbytes,
                   residual=dev(r, torch))
    torch.cuda.synchronize()
    check_tol(y.cpu().numpy(), y_ref, T, f"moe {fmt} N={N}")


def test_moe_full_shape_int4():
    """The MoE workload's shapes: H = 2048, 128 experts, I = 768, top-8 of
    seeded softmax logits, N = 8, int4 experts."""
    E, H, I, k, N = 128, 2048, 768, 8, 8
    bufs, Wgu, Wdn, xb, ids, gates, r = moe_case("int4", E, H, I, N, k, seed=77)
    y_ref, T = G.moe(G.x_from_bits(xb), ids, gates, Wgu, Wdn, r)
    nbytes = qg().moe_workspace_bytes(E, H, I, N, k)
    wsp = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((N, H), dtype=torch.float32, device="cuda")
    d = [dev(b, torch) for b in bufs]
    for _ in range(2):
        qg().qgemv_moe("int4", *d, E, H, I, dev(xb, torch), dev(ids, torch), dev(gates, torch), k, y, N, wsp,
                       nbytes, residual=dev(r, torch))
    torch.cuda.synchronize()
    check_tol(y.cpu().numpy(), y_ref, T, "moe full")


def test_moe_duplicates_and_bad_ids():
    E, H, I, k, N = 6, 128, 32, 3, 4
    ids = np.array([[0, 2, 2], [5, 1, 0], [3, 3, 3], [4, 0, 9]], np.int32)
    bufs, Wgu, Wdn, xb, ids, gates, r = moe_case("int5", E, H, I, N, k, seed=3, ids=ids)
    y_ref, T = G.moe(G.x_from_bits(xb), ids, gates, Wgu, Wdn, r)
    nbytes = qg().moe_workspace_bytes(E, H, I, N, k)
    wsp = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((N, H), dtype=torch.float32, device="cuda")
    d = [dev(b, torch) for b in bufs]
    qg().qgemv_moe("int5", *d, E, H, I, dev(xb, torch), dev(ids, torch), dev(gates, torch), k, y, N, wsp, nbytes,
                   residual=dev(r, torch))
    torch.cuda.synchronize()
    check_tol(y.cpu().numpy(), y_ref, T, "moe dup/bad")


@pytest.mark.parametrize("E,ids", [(3000, None),
                                   (5000, [[4999, 0, 2048, 4999], [2047, 2049, 4095, 4096], [1, 4998, 3, 2], [4999, 7, 4096, 0]])])
def test_moe_many_experts(E, ids):
    """Expert counts past one bitmap word per lane (E > 2048), with ids at the
    word edges and the last expert, so every slot's expert lookup is exercised."""
    H, I, k, N = 128, 32, 4, 4
    log("moe many experts", E)
    ids = None if ids is None else np.array(ids, np.int32)
    bufs, Wgu, Wdn, xb, ids, gates, r = moe_case("int4", E, H, I, N, k, seed=E, ids=ids)
    y_ref, T = G.moe(G.x_from_bits(xb), ids, gates, Wgu, Wdn, r)
    nbytes = qg().moe_workspace_bytes(E, H, I, N, k)
    wsp = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((N, H), dtype=torch.float32, device="cuda")
    d = [dev(b, torch) for b in bufs]
    qg().qgemv_moe("int4", *d, E, H, I, dev(xb, torch), dev(ids, torch), dev(gates, torch), k, y, N, wsp, nbytes,
                   residual=dev(r, torch))
    torch.cuda.synchronize()
    check_tol(y.cpu().numpy(), y_ref, T, f"moe E={E}")


@pytest.mark.parametrize("N,k,E", [(1, 8, 128), (8, 8, 128), (5, 3, 7), (8, 8, 4), (4, 3, 6), (8, 8, 3000), (3, 5, 1)])
def test_moe_index_bit_exact(N, k, E):
    rng = np.random.default_rng(N * 100 + k)
    ids = rng.integers(0, E, size=(N, k)).astype(np.int32)
    if E == 6:
        ids[0, 1] = -1
        ids[2, 2] = 99
    counts, offsets, pairs, active, n_active, err = G.moe_index(ids, E)
    t = [torch.full((n,), -7, dtype=torch.int32, device="cuda") for n in (E, E + 1, N * k, E, 2)]
    qg().qgemv_moe_index(dev(ids, torch), N, k, E, *t)
    torch.cuda.synchronize()
    g = [x.cpu().numpy() for x in t]
    assert np.array_equal(g[0], counts) and np.array_equal(g[1], offsets)
    assert np.array_equal(g[2], pairs) and np.array_equal(g[3], active)
    assert g[4][0] == n_active and g[4][1] == err


# --------------------------------------------------- full sizes, sampled rows

# every launch shape the benchmark times: [17408][5120] (one tile per
# workgroup) at N = 1, 2, 4, 8 in each format, the QKV shape and the down
# projection (one tile and 4-8 waves per workgroup), whose long K stages
# activations through the LDS ring or the whole range; and 9 to 32 tokens
# (one slot; 17 to 32 as two launches)
FULL = [("int4", 7168, 5120, 1), ("int4", 7168, 5120, 8), ("int4", 7168, 5120, 4), ("int5", 5120, 17408, 1),
        ("int5", 5120, 17408, 8), ("nvfp4", 5120, 17408, 4), ("nvfp4", 7168, 5120, 2),
        ("int4", 5120, 17408, 2), ("nvfp4", 5120, 17408, 2), ("int8", 5120, 17408, 2), ("int5", 5120, 17408, 3),
        ("int5", 17408, 5120, 16), ("int8", 7168, 5120, 12), ("int4", 5120, 17408, 16), ("int4", 17408, 5120, 32),
        ("int8", 5120, 17408, 24), ("nvfp4", 17408, 5120, 16), ("nvfp4", 5120, 17408, 12),
        ("nvfp4", 7168, 5120, 32),
        # the medium-grid launch shapes: one tile, 4-8 waves (every format on
        # the QKV-like and the down-like grid)
        ("int5", 7168, 5120, 2), ("int8", 7168, 5120, 1), ("nvfp4", 7168, 5120, 8), ("int4", 5120, 17408, 1),
        ("int4", 5120, 17408, 8), ("int8", 5120, 17408, 1), ("int8", 5120, 17408, 4), ("nvfp4", 5120, 17408, 1),
        ("nvfp4", 5120, 17408, 8), ("nvfp4", 7168, 5120, 1)] + \
       [(f, 17408, 5120, n) for f in ("int4", "int5", "int8", "nvfp4") for n in (1, 2, 4, 8)]


@pytest.mark.parametrize("fmt,M,K,N", FULL)
def test_full_size_sampled_rows(fmt, M, K, N):
    """Full-size GEMV in the benchmark's launch configuration; the oracle
    recomputes a sample of row tiles from the same packed bytes."""
    log("full", fmt, M, K, N)
    rng = synthetic.rng_for(0, 4, M, K)
    W = synthetic.weights(rng, M, K)
    xb = synthetic.activations(rng, N, K, 0.01)
    wq, ws = qg().pack(fmt, W)
    y = torch.empty((N, M), dtype=torch.float32, device="cuda")
    qg().qgemv(fmt, dev(wq, torch), dev(ws, torch), dev(xb, torch), y, M, K, N)
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    x = G.x_from_bits(xb)
    RT = M // 16
    for rt in sorted({0, 1, RT // 2, RT - 1, *np.random.default_rng(1).integers(0, RT, 4).tolist()}):
        Wt = tile_rows(fmt, wq, ws, M, K, rt)
        yr = G.gemv(x, Wt)
        T = G.gemv_tolerance(x, Wt)
        check_tol(yg[:, rt * 16:(rt + 1) * 16], yr, T, f"tile {rt}")


@pytest.mark.parametrize("fmt,N", [("nvfp4", 12), ("nvfp4", 32), ("int5", 24), ("int4", 16), ("int8", 32)])
def test_swiglu_full_size_many_tokens(fmt, N):
    """Gate/up pairs [2 x 17408][5120] at 9 to 32 tokens (one slot; 17 to 32
    as two token blocks sharing each decoded weight operand), sampled tiles."""
    I, K = 17408, 5120
    log("swiglu full", fmt, N)
    rng = synthetic.rng_for(0, 6, I, K)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, 2 * I, K))
    xb = synthetic.activations(rng, N, K, 0.01)
    h = torch.full((N, I), float("nan"), dtype=torch.float32, device="cuda")
    qg().qgemv_swiglu(fmt, dev(wq, torch), dev(ws, torch), dev(xb, torch), h, I, K, N)
    torch.cuda.synchronize()
    hg = h.cpu().numpy()
    x = G.x_from_bits(xb)
    RT = I // 16
    for rt in sorted({0, RT // 2, RT - 1, *np.random.default_rng(N).integers(0, RT, 3).tolist()}):
        Wg = tile_rows(fmt, wq, ws, 2 * I, K, rt)
        Wu = tile_rows(fmt, wq, ws, 2 * I, K, RT + rt)
        ref, T = G.swiglu_from(G.gemv(x, Wg), G.gemv(x, Wu), G.gemv_tolerance(x, Wg), G.gemv_tolerance(x, Wu))
        check_tol(hg[:, rt * 16:(rt + 1) * 16], ref, T, f"tile {rt}")
