"""Pins for the oracle's GEMV, SwiGLU, MoE index/combine and router:
exact rational brute force, closed forms, special cases and independent
reformulations."""
import math
from fractions import Fraction

import numpy as np
import pytest

import synthetic
from oracle import encodings as enc
from oracle import gemv as G
from oracle import quant
from oracle.dequant import dequant


def _x(rng, N, K, outliers=0.0):
    return G.x_from_bits(synthetic.activations(rng, N, K, outliers))


@pytest.mark.parametrize("N", [1, 3, 8])
def test_gemv_fp64_against_exact_fractions(N):
    rng = np.random.default_rng(N)
    M, K = 64, 64
    W = dequant(quant.quantize(synthetic.weights(rng, M, K), "int4"))
    x = _x(rng, N, K)
    r = synthetic.residual(rng, N, M)
    y = G.gemv(x, W, r)
    for n in range(N):
        for m in range(M):
            ex = G.exact_dot(x[n], W[m]) + Fraction(float(r[n, m]))
            bound = K * 2.0 ** -52 * (float(np.abs(x[n]) @ np.abs(W[m])) + abs(float(r[n, m])))
            assert abs(Fraction(float(y[n, m])) - ex) <= Fraction(bound)


def test_gemv_orientation_and_special_cases():
    rng = np.random.default_rng(7)
    M, K = 48, 96                      # non-square: a transposed operand fails
    W = dequant(quant.quantize(synthetic.weights(rng, M, K), "int5"))
    # one-hot x selects column k of W for every output row
    for k in (0, 5, 95):
        x = np.zeros((1, K))
        x[0, k] = 1.0
        assert np.array_equal(G.gemv(x, W)[0], W[:, k].astype(np.float64))
    # all-ones x gives row sums
    assert np.allclose(G.gemv(np.ones((2, K)), W), W.astype(np.float64).sum(axis=1)[None, :], rtol=0, atol=1e-12)
    # zero weights: y == residual exactly
    r = synthetic.residual(rng, 3, M)
    assert np.array_equal(G.gemv(_x(rng, 3, K), np.zeros((M, K), np.float32), r), r.astype(np.float64))
    # token n only sees row n of x
    x = _x(rng, 4, K)
    y = G.gemv(x, W)
    for n in range(4):
        assert np.array_equal(G.gemv(x[n:n + 1], W)[0], y[n])


def test_tolerance_covers_fp32_accumulation():
    rng = np.random.default_rng(8)
    M, K = 256, 5120
    W = dequant(quant.quantize(synthetic.weights(rng, M, K), "nvfp4"))
    x = _x(rng, 4, K, outliers=0.01)
    y = G.gemv(x, W)
    T = G.gemv_tolerance(x, W)
    # sequential fp32 accumulation in the worst (natural) order
    acc = np.zeros((4, M), np.float32)
    x32 = x.astype(np.float32)
    for k in range(K):
        acc += x32[:, k:k + 1] * W[None, :, k]
    assert np.all(np.abs(acc - y) <= T)
    # and the tolerance is not vacuous: scaling one weight row by 1.3 fails it
    W2 = W.copy()
    W2[3] *= 1.3
    assert np.any(np.abs(G.gemv(x, W2) - y) > T)


def test_bf16_inputs_decode():
    bits = synthetic.bf16_bits(np.array([[1.0, -2.5, 3.140625, 1e-3]], np.float32))
    v = G.x_from_bits(bits)
    assert v[0, 0] == 1.0 and v[0, 1] == -2.5 and v[0, 2] == 3.140625
    assert abs(v[0, 3] - 1e-3) <= 1e-3 * 2 ** -8
    # round to nearest even: 1 + 2^-8 is a tie between 1 and 1 + 2^-7
    assert synthetic.bf16_bits(np.array([1 + 2 ** -8], np.float32))[0] == 0x3F80
    assert synthetic.bf16_bits(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 0x3F82


def test_silu_closed_forms():
    assert G.silu(np.array([0.0]))[0] == 0.0
    assert G.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert G.silu(np.array([-1.0]))[0] == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert G.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert abs(G.silu(np.array([-40.0]))[0]) < 1e-15
    # the derivative bound used by the SwiGLU tolerance
    g = np.linspace(-20, 20, 200001)
    ds = np.gradient(G.silu(g), g)
    assert ds.max() < 1.1 and ds.min() > -0.11


def test_swiglu_uses_gate_rows_first():
    rng = np.random.default_rng(9)
    I, K = 32, 64
    W = dequant(quant.quantize(synthetic.weights(rng, 2 * I, K), "int4"))
    x = _x(rng, 2, K)
    h, Th = G.swiglu(x, W)
    g = x @ W[:I].astype(np.float64).T
    u = x @ W[I:].astype(np.float64).T
    assert np.allclose(h, g / (1 + np.exp(-g)) * u, rtol=1e-14, atol=0)
    h_swapped = u / (1 + np.exp(-u)) * g
    assert not np.allclose(h, h_swapped)
    assert np.all(Th > 0)


def test_moe_index_matches_stable_sort():
    rng = np.random.default_rng(10)
    for N, k, E in [(1, 8, 128), (8, 8, 128), (5, 3, 7), (8, 8, 4)]:
        ids = rng.integers(0, E, size=(N, k)).astype(np.int32)   # duplicates allowed
        counts, offsets, pairs, active, n_active, err = G.moe_index(ids, E)
        keys = sorted((int(ids[t, j]), t, j) for t in range(N) for j in range(k))
        assert [int(p) for p in pairs] == [t * k + j for (_, t, j) in keys]
        assert counts.sum() == N * k and offsets[-1] == N * k
        assert list(np.nonzero(counts)[0]) == list(active[:n_active])
        assert np.all(active[n_active:] == -1) and err == 0
        for e in range(E):
            seg = pairs[offsets[e]: offsets[e + 1]]
            assert all(ids.reshape(-1)[s] == e for s in seg)


def test_moe_index_flags_out_of_range_ids():
    ids = np.array([[0, 5, -1], [9, 2, 2]], np.int32)
    counts, offsets, pairs, active, n_active, err = G.moe_index(ids, 6)
    assert err == 1
    assert counts.sum() == 4 and offsets[-1] == 4
    assert list(pairs[:4]) == [0, 4, 5, 1] and list(pairs[4:]) == [-1, -1]
    assert list(active[:n_active]) == [0, 2, 5]


def test_moe_reference_equals_dense_expert_formulation():
    """sum over slots (the oracle) == sum over all experts weighted by a dense
    token x expert gate matrix (an independent arrangement)."""
    rng = np.random.default_rng(12)
    H, I, E, k, N = 64, 32, 6, 3, 4
    Wgu = [dequant(quant.quantize(synthetic.weights(rng, 2 * I, H), "int4")) for _ in range(E)]
    Wdn = [dequant(quant.quantize(synthetic.weights(rng, H, I), "int4")) for _ in range(E)]
    x = _x(rng, N, H)
    ids = np.array([[0, 2, 2], [5, 1, 0], [3, 3, 3], [4, 0, 9]], np.int32)   # dup + invalid
    gates = synthetic.random_gates(rng, N, k)
    r = synthetic.residual(rng, N, H)
    y, T = G.moe(x, ids, gates, Wgu, Wdn, r)
    Gm = np.zeros((N, E))
    for t in range(N):
        for j in range(k):
            if 0 <= ids[t, j] < E:
                Gm[t, ids[t, j]] += gates[t, j]
    dense = r.astype(np.float64).copy()
    for e in range(E):
        g = x @ Wgu[e][:I].astype(np.float64).T
        u = x @ Wgu[e][I:].astype(np.float64).T
        o = (g / (1 + np.exp(-g)) * u) @ Wdn[e].astype(np.float64).T
        dense += Gm[:, e:e + 1] * o
    assert np.allclose(y, dense, rtol=1e-12, atol=1e-12)
    assert np.all(T > 0)


def test_router_topk_softmax():
    rng = np.random.default_rng(13)
    logits = synthetic.router_logits(rng, 8, 128)
    logits[0, 10] = logits[0, 11] = 9.0            # a tie: lower index first
    ids, gates = G.route_topk_softmax(logits, 8)
    assert ids[0, 0] == 10 and ids[0, 1] == 11
    for t in range(8):
        order = np.argsort(-logits[t].astype(np.float64), kind="stable")[:8]
        assert list(ids[t]) == list(order)
        full = np.exp(logits[t].astype(np.float64) - logits[t].max())
        full /= full.sum()
        renorm = full[ids[t]] / full[ids[t]].sum()
        assert np.allclose(gates[t], renorm, rtol=1e-6)
        assert abs(float(gates[t].astype(np.float64).sum()) - 1.0) < 1e-6


def _beats(a, ia, b, ib):
    """True if logit a at index ia ranks above logit b at index ib: larger
    number first, equal numbers by lower index, NaN below every number."""
    na, nb = np.isnan(a), np.isnan(b)
    if na or nb:
        return (not na and nb) or (na and nb and ia < ib)
    return a > b or (a == b and ia < ib)


def test_router_selection_by_pairwise_rank():
    """The router's selection equals the experts whose pairwise rank (number
    of experts that beat them) is below k, in rank order; covers ties,
    -0/+0, infinities and NaNs."""
    rng = np.random.default_rng(17)
    rows = [
        np.array([1.0, np.nan, 3.0, -np.inf, 3.0, -0.0, 0.0, np.inf, np.nan, -2.0], np.float32),
        np.zeros(10, np.float32),
        np.full(10, np.nan, np.float32),
        rng.integers(-2, 3, 10).astype(np.float32),
    ]
    for row in rows:
        E = row.size
        for k in (1, 3, E):
            ids, _ = G.route_topk_softmax(row[None, :], k)
            rank = [sum(_beats(row[f], f, row[e], e) for f in range(E)) for e in range(E)]
            want = sorted((e for e in range(E) if rank[e] < k), key=lambda e: rank[e])
            assert list(ids[0]) == want, (row, k)
    ids, _ = G.route_topk_softmax(rows[0][None, :], 10)
    assert list(ids[0]) == [7, 2, 4, 0, 5, 6, 9, 3, 1, 8]


def test_router_tolerance_covers_fp32_and_rejects_larger_errors():
    rng = np.random.default_rng(19)
    logits = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    ids, g = G.route_topk_softmax(logits, 8)
    sel = np.take_along_axis(logits, ids.astype(np.int64), 1)
    # an fp32 evaluation in the stated order
    d = (sel - sel[:, :1]).astype(np.float32)
    e = np.exp(d).astype(np.float32)
    S = np.zeros(64, np.float32)
    for j in range(8):
        S = (S + e[:, j]).astype(np.float32)
    p32 = (e / S[:, None]).astype(np.float32)
    sel64 = sel.astype(np.float64)
    ref = np.exp(sel64 - sel64[:, :1])
    ref /= ref.sum(1, keepdims=True)
    T = G.route_tolerance(logits, ids, ref)
    assert np.all(np.abs(p32 - ref) <= T)
    assert np.all(np.abs(g - ref) <= T)            # the oracle's own fp32 rounding
    assert np.all(T < 1e-4 * ref + 1e-10)          # and the bound stays tight
    bad = p32 * np.float32(1 + 2e-4)
    assert np.any(np.abs(bad - ref) > T)


def test_rmsnorm_closed_forms():
    # h = [3, 4]: mean square 12.5, so x = h / sqrt(12.5) (hand-worked)
    x = G.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    assert np.allclose(x, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)
    assert abs(float(np.mean(x * x)) - 1.0) < 1e-15          # unit mean square
    # a constant row normalises to sign(c) * gamma (eps = 0), gamma applied per column
    g = np.linspace(-2, 3, 16)
    assert np.allclose(G.rmsnorm(np.full((1, 16), -7.5), g, 0.0), -g[None, :], rtol=1e-15)
    # scale invariance (eps = 0) and rows independent
    rng = np.random.default_rng(31)
    h = rng.standard_normal((3, 64))
    assert np.allclose(G.rmsnorm(h * 1e3, g.repeat(4), 0.0), G.rmsnorm(h, g.repeat(4), 0.0), rtol=1e-13)
    assert np.allclose(G.rmsnorm(h[1:2], g.repeat(4), 1e-5), G.rmsnorm(h, g.repeat(4), 1e-5)[1:2], rtol=0)
    # eps enters under the square root of the mean square
    x = G.rmsnorm(np.array([[1.0, 1.0]]), np.ones(2), 3.0)
    assert np.allclose(x, [[0.5, 0.5]], rtol=1e-15)


def test_norm_tolerance_covers_the_gpu_evaluation():
    """An fp32 emulation of the normalised GEMV the GPU runs (bf16(gamma*h)
    operands, fp32 dot, fp32 norm scale applied after) stays within the
    bound; planted mistakes (sum instead of mean, gamma applied twice, no
    scale) do not."""
    rng = np.random.default_rng(33)
    N, K, M = 4, 5120, 96
    W = dequant(quant.quantize(synthetic.weights(rng, M, K), "int5"))
    h = rng.standard_normal((N, K)).astype(np.float32) * np.float32(3)
    gamma = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    x = G.rmsnorm(h, gamma, 1e-6)
    y_ref = G.gemv(x, W)
    T = G.norm_gemv_tolerance(x, W)

    def emul(scale_fn, gmul=1):
        a = enc.f32_from_bf16_bits(synthetic.bf16_bits((h * (gamma * np.float32(gmul))).astype(np.float32)))
        dot = (a.astype(np.float32) @ W.astype(np.float32).T).astype(np.float32)
        ss = np.sum(h * h, axis=1, dtype=np.float32)
        return (dot * scale_fn(ss)[:, None]).astype(np.float64)
    good = emul(lambda ss: (np.float32(1) / np.sqrt(ss / np.float32(K) + np.float32(1e-6))).astype(np.float32))
    assert np.all(np.abs(good - y_ref) <= T)
    bad_sum = emul(lambda ss: (np.float32(1) / np.sqrt(ss + np.float32(1e-6))).astype(np.float32))
    bad_gamma = emul(lambda ss: (np.float32(1) / np.sqrt(ss / np.float32(K) + np.float32(1e-6))).astype(np.float32),
                     gmul=gamma)
    no_scale = emul(lambda ss: np.ones_like(ss))
    for bad in (bad_sum, bad_gamma, no_scale):
        assert np.any(np.abs(bad - y_ref) > T)


# ------------------------------------------- pins of the propagated bounds
#
# Sign-coherent inputs (every product x_k w_k of a row has the row's sign)
# make sum|x w| = |sum x w|, so the GEMV bound is 2e-3 of the value itself
# and a propagated bound that came out too loose by a plausible typo (a
# factor 10 or 100) lets the planted mistakes below through.

def _coherent(rng, rows, K, signs, scale):
    """[rows][K] fp32 weights whose row r has the sign signs[r] throughout."""
    w = rng.uniform(0.2, 1.8, (rows, K)) * scale / K
    return (w * np.asarray(signs, np.float64)[:, None]).astype(np.float32)


def _f32_dot(x, W):
    """fp32 emulation of a GPU dot: fp32 products summed sequentially in fp32."""
    x32, W32 = np.asarray(x, np.float32), np.asarray(W, np.float32)
    acc = np.zeros((x32.shape[0], W32.shape[0]), np.float32)
    for k in range(x32.shape[1]):
        acc += x32[:, k:k + 1] * W32[None, :, k]
    return acc


def _f32_silu_mul(g, u):
    g, u = np.asarray(g, np.float32), np.asarray(u, np.float32)
    with np.errstate(over="ignore"):
        return (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float32)


def _swiglu_case(seed=41, N=3, K=256, I=48):
    rng = np.random.default_rng(seed)
    x = G.x_from_bits(synthetic.bf16_bits(rng.uniform(0.5, 1.5, (N, K)).astype(np.float32)))
    gs = np.where(np.arange(I) % 3 == 0, -1.0, 1.0)           # gates of both signs
    Wg = _coherent(rng, I, K, gs, rng.uniform(0.3, 4.0, I)[:, None])
    Wu = _coherent(rng, I, K, np.where(np.arange(I) % 4 == 1, -1.0, 1.0), rng.uniform(0.5, 3.0, I)[:, None])
    return x, np.concatenate([Wg, Wu])


def test_swiglu_bound_contains_the_gpu_evaluation_and_rejects_mistakes():
    x, W = _swiglu_case()
    I = W.shape[0] // 2
    h, Th = G.swiglu(x, W)
    g, u = G.gemv(x, W[:I]), G.gemv(x, W[I:])
    Tg, Tu = G.gemv_tolerance(x, W[:I]), G.gemv_tolerance(x, W[I:])
    # the GPU's evaluation: fp32 dots, then fp32 silu(g) * u
    h32 = _f32_silu_mul(_f32_dot(x, W[:I]), _f32_dot(x, W[I:]))
    assert np.all(np.abs(h32 - h) <= Th)
    # worst-case inputs: g and u anywhere inside their own bounds
    for sg in (-1, 1):
        for su in (-1, 1):
            hw = G.silu(g + sg * 0.999 * Tg) * (u + su * 0.999 * Tu)
            assert np.all(np.abs(hw - h) <= Th)
    # the bound is tight: a few times 2e-3 of |h| where silu(g) is not small
    # against g (g > 0.5: silu(g) / g > 0.62)
    big = g > 0.5
    assert np.all(Th[big] <= 0.012 * np.abs(h[big]) + 2e-5)
    # planted mistakes fall outside it
    mistakes = {
        "gate and up swapped": G.silu(u) * g,
        "sigmoid instead of silu": g * 0 + 1.0 / (1.0 + np.exp(-g)) * u,
        "gate row off by one": G.silu(np.roll(g, 1, axis=1)) * u,
        "h scaled by 1.01": h * 1.01,
        "silu(-g)": G.silu(-g) * u,
    }
    for what, bad in mistakes.items():
        assert np.any(np.abs(bad - h) > Th), what


def _moe_case(seed=43, N=2, H=64, I=32, E=3, k=2):
    rng = np.random.default_rng(seed)
    x = G.x_from_bits(synthetic.bf16_bits(rng.uniform(0.5, 1.5, (N, H)).astype(np.float32)))
    Wgu = [np.concatenate([_coherent(rng, I, H, np.ones(I), rng.uniform(0.5, 3.0, I)[:, None]),
                           _coherent(rng, I, H, np.ones(I), rng.uniform(0.5, 3.0, I)[:, None])]) for _ in range(E)]
    Wdn = [_coherent(rng, H, I, np.ones(H), 2.0) for _ in range(E)]
    ids = np.array([[0, 2], [1, 0]], np.int32)[:N, :k]
    gates = np.array([[0.625, 0.375], [0.55, 0.45]], np.float32)[:N, :k]
    return x, Wgu, Wdn, ids, gates


def test_moe_bound_contains_the_gpu_evaluation_and_rejects_mistakes():
    x, Wgu, Wdn, ids, gates = _moe_case()
    N, k = ids.shape
    I = Wgu[0].shape[0] // 2
    y, T = G.moe(x, ids, gates, Wgu, Wdn)

    def run(h_of, p_of=lambda t, j: float(gates[t, j]), e_of=lambda t, j: int(ids[t, j]), slots=range(k)):
        out = np.zeros_like(y)
        for t in range(N):
            for j in slots:
                e = e_of(t, j)
                out[t] += p_of(t, j) * (h_of(t, e) @ np.asarray(Wdn[e], np.float64).T)[0]
        return out

    def h_exact(t, e):
        return G.swiglu(x[t:t + 1], Wgu[e])[0]

    # the GPU's evaluation: fp32 h, kept as a bf16 hi/lo pair, fp32 down dot,
    # fp32 fused multiply-adds of the mixing weights in slot order
    y32 = np.zeros(y.shape, np.float32)
    for t in range(N):
        for j in range(k):
            e = int(ids[t, j])
            h32 = _f32_silu_mul(_f32_dot(x[t:t + 1], Wgu[e][:I]), _f32_dot(x[t:t + 1], Wgu[e][I:]))
            hi = enc.f32_from_bf16_bits(synthetic.bf16_bits(h32))
            lo = enc.f32_from_bf16_bits(synthetic.bf16_bits((h32 - hi).astype(np.float32)))
            o32 = (_f32_dot(hi, Wdn[e]) + _f32_dot(lo, Wdn[e])).astype(np.float32)
            y32[t] = (np.float64(gates[t, j]) * o32[0] + y32[t]).astype(np.float32)
    assert np.all(np.abs(y32 - y) <= T)
    # worst case: h anywhere inside its own bound, then the down GEMV's 2e-3
    for s in (-1, 1):
        def h_worst(t, e, s=s):
            hh, Th = G.swiglu(x[t:t + 1], Wgu[e])
            return hh + s * 0.999 * Th
        yw = run(h_worst)
        assert np.all(np.abs(yw - y) + 0.999 * G.REL * np.abs(yw) <= T)
    # the bound is tight: under 1% of |y| on these sign-coherent inputs
    assert np.all(T <= 0.01 * np.abs(y))
    # planted mistakes fall outside it
    other = {0: 1, 1: 2, 2: 0}
    mistakes = {
        "mixing weights off by 1%": run(h_exact, p_of=lambda t, j: 1.01 * float(gates[t, j])),
        "one slot dropped": run(h_exact, slots=range(k - 1)),
        "wrong expert in one slot": run(h_exact, e_of=lambda t, j: other[int(ids[t, j])] if (t, j) == (0, 1)
                                        else int(ids[t, j])),
        "gate and up swapped": run(lambda t, e: (G.silu(G.gemv(x[t:t + 1], Wgu[e][I:]))
                                                 * G.gemv(x[t:t + 1], Wgu[e][:I]))),
        "unweighted sum of slots": run(h_exact, p_of=lambda t, j: 1.0 / k),
    }
    for what, bad in mistakes.items():
        assert np.any(np.abs(bad - y) > T), what


def test_chain_bound_contains_a_bf16_hand_off_and_rejects_mistakes():
    """h (a SwiGLU output within T_h) crosses to the down projection as bf16."""
    x, W = _swiglu_case(seed=45)
    I = W.shape[0] // 2
    rng = np.random.default_rng(46)
    Wd = _coherent(rng, 40, I, np.ones(40), 1.5)
    h, Th = G.swiglu(x, W)
    y = G.gemv(h, Wd)
    T = G.chain_tolerance(h, Th, Wd)

    def bf16(v):
        return enc.f32_from_bf16_bits(synthetic.bf16_bits(np.asarray(v, np.float32))).astype(np.float64)
    # the GPU's evaluation: fp32 h, rounded to bf16, fp32 down dot
    h32 = _f32_silu_mul(_f32_dot(x, W[:I]), _f32_dot(x, W[I:]))
    assert np.all(np.abs(_f32_dot(bf16(h32), Wd) - y) <= T)
    # worst case: h at the edge of its bound, rounded to bf16, down GEMV at its own 2e-3
    for s in (-1, 1):
        hw = bf16(h + s * 0.999 * Th)
        yw = G.gemv(hw, Wd)
        assert np.all(np.abs(yw - y) + 0.999 * G.REL * (np.abs(hw) @ np.abs(Wd).T) <= T)
    mistakes = {
        "h rounded to fp8 e4m3 instead of bf16": G.gemv(enc.e4m3_decode(
            np.array([[enc.exact_e4m3_bits(enc.exact_round_e4m3_sat(Fraction(float(v)))) if v >= 0 else 0 for v in row]
                      for row in h],
                     np.uint8)), Wd),
        "silu(g) handed over without u": G.gemv(G.silu(G.gemv(x, W[:I])), Wd),
        "h scaled by 1.02": y * 1.02,
    }
    for what, bad in mistakes.items():
        assert np.any(np.abs(bad - y) > T), what
