"""GPU parity on adversarial weights and exact special cases, through the C ABI.

* int4 / int5 groups chosen to stress the group scale step (a weight of
  c + q with c the code bias, and d * (D - Db) + (m / c) * Db): groups whose
  weights are all zero but one, met by an activation 20 to 100 times
  smaller than its neighbours; groups with m = -d * q0 so that most weights are zero or
  tiny; large d with an fp16 subnormal m; rows whose groups differ by many
  orders of magnitude. Built with qgemv_pack_codes from codes and scale
  fields, checked per output against the oracle's bound,
  2e-3 sum|x w| + 1e-5. With activations 10^3 to 10^4 times smaller at the
  single nonzero weight, the code bias can carry the error past that bound;
  those cases are checked against the bound the kernel's arithmetic gives
  (decode_bias_bound).
* One-hot activations of value 2^j: every sum the kernel forms is then exact,
  so y equals 2^j times the dequantised weight column bit for bit (up to
  the sign of zero), in every format, at several token counts, with and
  without the split-remainder workspace.
* The MoE routing index through each path's own routine (qgemv_moe's
  per-slot routing and the single launch's lane ranking), bit for bit.
"""
import zlib

import numpy as np
import pytest

import synthetic
from gpu_helpers import FORMATS, check_tol, dev, oracle_weights, tile_rows
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


def f16_bits(v):
    return np.asarray(v, np.float16).view(np.uint16)


def adversarial_case(kind, fmt, M, K, N, seed, hot_scale=0.05):
    """codes [M][K], d bits, m bits (fp16) and bf16 x [N][K] for one kind;
    hot_scale: the activation magnitude (times 0.5 to 1.5, either sign)
    where a single-nonzero group's nonzero weight sits; the others are
    N(0, 1)."""
    rng = np.random.default_rng(seed)
    G_ = K // 32
    qmax = 15 if fmt == "int4" else 31
    x = rng.standard_normal((N, K)).astype(np.float32)
    codes = np.zeros((M, K), np.uint8)
    if kind == "single_nonzero":
        # all codes q0 with d * q0 + m = 0 exactly (d has few significant
        # bits, so d * q0 is an exact fp16), one other code per group; the
        # activation at that position is small
        d = (rng.integers(1, 64, (M, G_)) * 2.0 ** rng.integers(-12, -2, (M, G_))).astype(np.float16)
        q0 = np.where(rng.random((M, G_)) < 0.5, 0, qmax).astype(np.int64)
        m = (-(d.astype(np.float64) * q0)).astype(np.float16)
        codes[:] = np.repeat(q0, 32, axis=1)
        for r in range(M):
            for g in range(G_):
                j = 32 * g + int(rng.integers(0, 32))
                codes[r, j] = int(rng.integers(1, qmax)) if q0[r, g] == 0 else int(rng.integers(0, qmax - 1))
        hot = rng.integers(0, 32, G_)
        for g in range(G_):                       # small x where every row's nonzero code sits
            x[:, 32 * g + hot[g]] = hot_scale * rng.choice([-1.0, 1.0], N) * rng.uniform(0.5, 1.5, N)
        # and make every row's nonzero code sit at those positions
        for r in range(M):
            for g in range(G_):
                seg = codes[r, 32 * g:32 * g + 32]
                nz = int(np.nonzero(seg != q0[r, g])[0][0])
                seg[nz], seg[hot[g]] = seg[hot[g]], seg[nz]
    elif kind == "centered":
        # m = -d * qbar (rounded to fp16): weights d (q - qbar) with q near qbar
        d = rng.uniform(1e-3, 0.5, (M, G_)).astype(np.float16)
        qbar = rng.integers(2, qmax - 1, (M, G_))
        m = (-(d.astype(np.float64) * (qbar + rng.uniform(-0.01, 0.01, (M, G_))))).astype(np.float16)
        q = np.repeat(qbar, 32, axis=1) + rng.integers(-2, 3, (M, K))
        codes[:] = np.clip(q, 0, qmax)
    elif kind == "big_d_subnormal_m":
        d = rng.uniform(256, 4096, (M, G_)).astype(np.float16)
        mb = rng.integers(1, 0x3FF, (M, G_)).astype(np.uint16) | np.where(rng.random((M, G_)) < 0.5, 0x8000, 0).astype(np.uint16)
        m = mb.view(np.float16)
        codes[:] = rng.integers(0, qmax + 1, (M, K))
    elif kind == "mixed_magnitudes":
        d = (rng.uniform(1, 2, (M, G_)) * 2.0 ** rng.integers(-14, 11, (M, G_))).astype(np.float16)
        m = (-(d.astype(np.float64) * rng.uniform(0, qmax, (M, G_)))).astype(np.float16)
        codes[:] = rng.integers(0, qmax + 1, (M, K))
    else:
        raise ValueError(kind)
    assert np.all(np.isfinite(d)) and np.all(np.isfinite(m))
    xb = synthetic.bf16_bits(x)
    return codes, f16_bits(d), f16_bits(m), xb


KINDS = ["single_nonzero", "centered", "big_d_subnormal_m", "mixed_magnitudes"]


@pytest.mark.parametrize("fmt", ["int4", "int5"])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("K", [32, 160, 5120])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
def test_adversarial_int_groups(fmt, kind, K, N):
    M = 48
    log("adversarial", fmt, kind, K, N)
    hot = 0.01 if N in (2, 8) else 0.05      # activation at the single nonzero weight: 100x / 20x smaller
    codes, d, m, xb = adversarial_case(kind, fmt, M, K, N, seed=zlib.crc32(f"{fmt} {kind} {K} {N}".encode()),
                                       hot_scale=hot)
    wq, ws = qg().pack_codes(fmt, codes, d, m)
    y = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda")
    qg().qgemv(fmt, dev(wq, torch), dev(ws, torch), dev(xb, torch), y, M, K, N)
    torch.cuda.synchronize()
    W = oracle_weights(fmt, wq, ws, M, K)
    x = G.x_from_bits(xb)
    r = check_tol(y.cpu().numpy(), G.gemv(x, W), G.gemv_tolerance(x, W), f"{fmt} {kind} K={K} N={N}")
    log(f"  max err/tol {r:.3g}")


def decode_bias_bound(fmt, x, codes, d_bits, m_bits, T):
    """The device bound of the int group step: the contract bound T plus
    2^-18 * sum_g (c |d_g| + |m_g|) * sum_{k in g} |x_k| per output, c the
    code bias (16 int4, 32 int5). It follows from the bf16 MFMA's arithmetic
    as measured on gfx950 (each 8-product block aligned to its largest
    product and truncated to a 25-bit window, blocks then added in fp32):
    D = sum x (c + q) and Db = c sum x each carry under 2^-20 c sum|x| per
    block in truncation and conversion and 2^-22 c sum|x| in the block
    additions, so D - Db errs by under 2^-18 c sum|x| per group; the m term
    carries Db's error times |m| / c."""
    c = 16.0 if fmt == "int4" else 32.0
    d = np.abs(d_bits.view(np.float16).astype(np.float64))
    m = np.abs(m_bits.view(np.float16).astype(np.float64))
    ax = np.abs(x).reshape(x.shape[0], -1, 32).sum(axis=2)           # [N][G]
    return T + 2.0 ** -18 * (ax @ (c * d + m).T)


@pytest.mark.parametrize("fmt", ["int4", "int5"])
@pytest.mark.parametrize("K", [32, 160])
@pytest.mark.parametrize("N", [1, 8])
@pytest.mark.parametrize("hot_scale", [1e-3, 1e-4])
def test_adversarial_decode_bias_limit(fmt, K, N, hot_scale):
    """Groups whose weights are all zero but one, where the activation is
    10^3 to 10^4 times smaller than its neighbours: the code bias c makes the
    MFMA sums carry truncation of order 2^-24 c d sum|x|, which can exceed
    2e-3 sum|x w| + 1e-5 there. The kernel stays within the bound derived
    from its arithmetic (decode_bias_bound); how far past the contract it
    goes is printed."""
    M = 48
    log("decode-bias limit", fmt, K, N, hot_scale)
    codes, d, m, xb = adversarial_case("single_nonzero", fmt, M, K, N,
                                       seed=zlib.crc32(f"limit {fmt} {K} {N} {hot_scale}".encode()),
                                       hot_scale=hot_scale)
    wq, ws = qg().pack_codes(fmt, codes, d, m)
    y = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda")
    qg().qgemv(fmt, dev(wq, torch), dev(ws, torch), dev(xb, torch), y, M, K, N)
    torch.cuda.synchronize()
    W = oracle_weights(fmt, wq, ws, M, K)
    x = G.x_from_bits(xb)
    yr, T = G.gemv(x, W), G.gemv_tolerance(x, W)
    yg = y.cpu().numpy().astype(np.float64)
    check_tol(yg, yr, decode_bias_bound(fmt, x, codes, d, m, T), f"{fmt} K={K} N={N} hot={hot_scale}")
    log(f"  err / contract bound: max {float((np.abs(yg - yr) / T).max()):.3g}")


def _same_values(got, want):
    """Equal as numbers (so -0 == +0), and equal bits wherever nonzero."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    ok = (got == want) | (np.isnan(got) & np.isnan(want))
    nz = want != 0
    ok &= ~nz | (got.view(np.uint32) == want.view(np.uint32))
    return ok


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,K", [(48, 256), (100, 5120)])
@pytest.mark.parametrize("N", [1, 2, 3, 8, 16])
def test_one_hot_equals_dump_bit_exact(fmt, M, K, N):
    """Token t has one activation 2^j at column k_t: y[t] = 2^j * W[:, k_t]."""
    log("one-hot", fmt, M, K, N)
    rng = synthetic.rng_for(8, M, K, N)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, M, K))
    W = oracle_weights(fmt, wq, ws, M, K)
    ks = rng.choice(K, N, replace=False)
    pw = rng.integers(-2, 3, N)
    x = np.zeros((N, K), np.float32)
    x[np.arange(N), ks] = 2.0 ** pw
    y = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda")
    qg().qgemv(fmt, dev(wq, torch), dev(ws, torch), dev(synthetic.bf16_bits(x), torch), y, M, K, N)
    torch.cuda.synchronize()
    want = (W[:, ks].T.astype(np.float64) * 2.0 ** pw[:, None]).astype(np.float32)
    ok = _same_values(y.cpu().numpy(), want)
    assert ok.all(), np.argwhere(~ok)[:5]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N", [1, 8])
def test_one_hot_bit_exact_with_split_remainder(fmt, N):
    """[17408][5120] with the split-remainder workspace (the fragments' partial
    sums meet in the workspace): still the dump column, on sampled tiles."""
    M, K = 17408, 5120
    log("one-hot split", fmt, N)
    rng = synthetic.rng_for(9, M, K, N)
    wq, ws = qg().pack(fmt, synthetic.weights(rng, M, K))
    ks = rng.choice(K, N, replace=False)
    x = np.zeros((N, K), np.float32)
    x[np.arange(N), ks] = 1.0
    y = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda")
    wsp = qg().split_workspace("cuda")
    qg().qgemv_ex(fmt, dev(wq, torch), dev(ws, torch), dev(synthetic.bf16_bits(x), torch), y, M, K, N,
                  workspace=wsp)
    qg().check_split_workspace(wsp)
    yg = y.cpu().numpy()
    RT = M // 16
    for rt in sorted({0, RT - 1, RT - 5, RT - 40, *np.random.default_rng(2).integers(0, RT, 3).tolist()}):
        Wt = tile_rows(fmt, wq, ws, M, K, rt)
        ok = _same_values(yg[:, rt * 16:(rt + 1) * 16], Wt[:, ks].T)
        assert ok.all(), (rt, np.argwhere(~ok)[:5])


def _index_cases():
    cases = [(1, 8, 128, None), (8, 8, 128, None), (5, 3, 7, None), (8, 8, 4, None), (4, 3, 6, "bad"),
             (8, 8, 3000, None), (3, 5, 1, None), (8, 8, 16384, None), (8, 8, 16384, "edges"), (2, 8, 1, "bad"),
             (8, 8, 64, "dups"), (1, 1, 1, None), (7, 1, 5, "bad")]
    return cases


@pytest.mark.parametrize("routine", [0, 1])
@pytest.mark.parametrize("N,k,E,mod", _index_cases())
def test_moe_index_by_routine_bit_exact(routine, N, k, E, mod):
    rng = np.random.default_rng(N * 1000 + k * 10 + E % 97)
    ids = rng.integers(0, E, size=(N, k)).astype(np.int32)
    if mod == "bad":
        ids[0, 0] = -1
        ids[-1, -1] = E + 3
    elif mod == "edges":
        ids[:, :4] = np.array([0, E - 1, 8191, 8192])
    elif mod == "dups":
        ids[:] = rng.integers(0, 3, size=(N, k))
    counts, offsets, pairs, active, n_active, err = G.moe_index(ids, E)
    t = [torch.full((n,), -7, dtype=torch.int32, device="cuda") for n in (E, E + 1, N * k, E, 2)]
    qg().qgemv_moe_index_by(routine, dev(ids, torch), N, k, E, *t)
    torch.cuda.synchronize()
    g = [x.cpu().numpy() for x in t]
    assert np.array_equal(g[0], counts) and np.array_equal(g[1], offsets)
    assert np.array_equal(g[2], pairs) and np.array_equal(g[3], active)
    assert g[4][0] == n_active and g[4][1] == err
