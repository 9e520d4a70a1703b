"""GPU parity of the device MoE router (qgemv_moe_route) and the single-launch
MoE (qgemv_moe_fused) against the oracle, through the C ABI.

Bit-exact: the selected expert ids (the oracle's top-k order: larger logit
first, ties to the lower index, NaN last). Tolerance: the mixing weights
within oracle.gemv.route_tolerance; the MoE output within the oracle's MoE
bound widened by the weights' tolerance. With more than 8 routed rows the fused
call runs the router and then qgemv_moe's launches, so the two give identical
bits on the same ids and weights; with 8 or fewer it is one launch of its own,
checked against the oracle and for run-to-run determinism.
"""
import numpy as np
import pytest

import synthetic
from gpu_helpers import FORMATS, check_tol, dev, moe_case
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


def _route_gpu(logits, k):
    N, E = logits.shape
    ids = torch.full((N, k), -7, dtype=torch.int32, device="cuda")
    gates = torch.full((N, k), float("nan"), dtype=torch.float32, device="cuda")
    qg().qgemv_moe_route(dev(logits, torch), N, E, k, ids, gates)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), gates.cpu().numpy()


def _ref_gates(logits, ids):
    sel = np.take_along_axis(np.asarray(logits, np.float64), ids.astype(np.int64), 1)
    g = np.exp(sel - sel[:, :1])
    return g / g.sum(1, keepdims=True)


@pytest.mark.parametrize("N,E,k", [(1, 128, 8), (8, 128, 8), (3, 7, 3), (37, 64, 1), (5, 300, 8), (2, 1000, 2),
                                   (4, 16384, 8), (6, 65, 64), (9, 8, 8)])
def test_route_parity(N, E, k):
    log("route", N, E, k)
    rng = synthetic.rng_for(11, N, E, k)
    logits = synthetic.router_logits(rng, N, E) * np.float32(3)
    ids_ref, _ = G.route_topk_softmax(logits, k)
    ids, gates = _route_gpu(logits, k)
    assert np.array_equal(ids, ids_ref), np.argwhere(ids != ids_ref)[:5]
    ref = _ref_gates(logits, ids_ref)
    T = G.route_tolerance(logits, ids_ref, ref)
    check_tol(gates, ref, T, "gates")


def test_route_ties_zeros_infinities_nans():
    """Rows of equal logits, -0/+0, +-inf and NaNs: ids bit-exact against the
    oracle's ordering; weights checked where the selected logits are finite."""
    rows = np.array([
        [1.0, np.nan, 3.0, -np.inf, 3.0, -0.0, 0.0, np.inf, np.nan, -2.0, 3.0, 1.0],
        [0.0] * 12,
        [np.nan] * 12,
        [-0.0, 0.0] * 6,
        [5.0, 5.0, 5.0, -1.0, -1.0, 2.0, 2.0, 2.0, 2.0, 7.0, -np.inf, 5.0],
    ], np.float32)
    for k in (1, 4, 12):
        ids_ref, _ = G.route_topk_softmax(rows, k)
        ids, gates = _route_gpu(rows, k)
        assert np.array_equal(ids, ids_ref), (k, ids, ids_ref)
        for t in (1, 3, 4):
            if t == 4 and k == 12:
                continue                                  # -inf selected: weight 0, checked below
            ref = _ref_gates(rows[t:t + 1], ids_ref[t:t + 1])
            check_tol(gates[t:t + 1], ref, G.route_tolerance(rows[t:t + 1], ids_ref[t:t + 1], ref), f"k={k} t={t}")
    ids, gates = _route_gpu(rows[4:5], 12)
    assert gates[0, -1] == 0.0 and abs(float(gates[0].astype(np.float64).sum()) - 1.0) < 1e-6


def test_route_rejects_bad_arguments():
    x = torch.zeros((2, 8), dtype=torch.float32, device="cuda")
    i = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    g = torch.zeros((2, 8), dtype=torch.float32, device="cuda")
    lib = qg().load()
    s = torch.cuda.current_stream().cuda_stream
    assert lib.qgemv_moe_route(x.data_ptr(), 2, 8, 9, i.data_ptr(), g.data_ptr(), s) == -7   # top_k > E
    assert lib.qgemv_moe_route(None, 2, 8, 2, i.data_ptr(), g.data_ptr(), s) == -1
    assert lib.qgemv_moe_route(x.data_ptr(), 0, 8, 2, i.data_ptr(), g.data_ptr(), s) == -1


# ------------------------------------------------------------ fused MoE

def _fused_case(fmt, E, H, I, N, k, seed, logits=None):
    if logits is None:
        rng = synthetic.rng_for(12, seed, E, N)
        logits = synthetic.router_logits(rng, N, E) * np.float32(2)
    bufs, Wgu, Wdn, xb, ids, gates, r = moe_case(fmt, E, H, I, N, k, seed=seed, logits=logits)
    return logits, bufs, Wgu, Wdn, xb, ids, gates, r


def _run_fused(fmt, bufs, E, H, I, xb, logits, k, N, r, wsp=None, calls=1):
    nbytes = qg().moe_fused_workspace_bytes(E, H, I, N, k)
    if wsp is None:
        wsp = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    d = [dev(b, torch) for b in bufs]
    y = torch.full((N, H), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((N, k), -7, dtype=torch.int32, device="cuda")
    gates = torch.full((N, k), float("nan"), dtype=torch.float32, device="cuda")
    out = []
    for _ in range(calls):
        qg().qgemv_moe_fused(fmt, *d, E, H, I, dev(xb, torch), dev(logits, torch), k, y, N, wsp, nbytes,
                             residual=None if r is None else dev(r, torch), ids_out=ids, gates_out=gates)
        torch.cuda.synchronize()
        out.append(y.cpu().numpy().copy())
    w = wsp.cpu().numpy().view(np.uint32)
    return out, ids.cpu().numpy(), gates.cpu().numpy(), w, d


def _check_flags(w, I, N, k, ids):
    """The fused workspace's head: the sticky error word (byte 12) and the
    64-bit item flags [8 slots][I / 16 row blocks] from byte 256. After calls
    on a fresh workspace, every item of an active slot holds the last call's
    number and nothing else was written; with more than 8 routed rows the
    single launch does not run and the head stays zero."""
    assert w[3] == 0, "a dependency wait timed out"
    assert np.all(w[:64] == 0), np.nonzero(w[:64])
    nA = (I + 15) // 16
    fl = w[64: 64 + 2 * 8 * nA].view(np.uint64).reshape(8, nA)
    if N * k > 8:
        assert np.all(fl == 0)
        return
    n_active = len(np.unique(ids))
    last = fl[0, 0]
    assert last > 0 and np.all(fl[:n_active] == last), fl[:n_active]
    assert np.all(fl[n_active:] == 0)


def _check_fused(fmt, E, H, I, N, k, seed, calls=2, logits=None):
    logits, bufs, Wgu, Wdn, xb, ids_ref, _, r = _fused_case(fmt, E, H, I, N, k, seed, logits)
    ys, ids, gates, w, d = _run_fused(fmt, bufs, E, H, I, xb, logits, k, N, r, calls=calls)
    assert np.array_equal(ids, ids_ref), (ids, ids_ref)
    _check_flags(w, I, N, k, ids)
    ref_g = _ref_gates(logits, ids_ref)
    Tg = G.route_tolerance(logits, ids_ref, ref_g)
    check_tol(gates, ref_g, Tg, "fused gates")
    ids_r, gates_r = _route_gpu(logits, k)                # the same router in its own launch
    assert np.array_equal(ids_r, ids) and np.array_equal(gates_r.view(np.uint32), gates.view(np.uint32))
    y_ref, T = G.moe(G.x_from_bits(xb), ids_ref, ref_g, Wgu, Wdn, r, gate_tol=Tg)
    for y in ys:
        check_tol(y, y_ref, T, f"fused moe {fmt} N={N}")
    for y in ys[1:]:
        assert np.array_equal(y.view(np.uint32), ys[0].view(np.uint32)), "repeat call differs"
    # the three-launch path on the same ids and weights: the same bits when the
    # fused call takes that path (N * top_k > 8), within tolerance otherwise
    nb = qg().moe_workspace_bytes(E, H, I, N, k)
    wsp2 = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    y2 = torch.empty((N, H), dtype=torch.float32, device="cuda")
    qg().qgemv_moe(fmt, *d, E, H, I, dev(xb, torch), dev(ids, torch), dev(gates, torch), k, y2, N, wsp2, nb,
                   residual=None if r is None else dev(r, torch))
    torch.cuda.synchronize()
    y2 = y2.cpu().numpy()
    if N * k > 8:
        assert np.array_equal(y2.view(np.uint32), ys[0].view(np.uint32)), np.argwhere(y2 != ys[0])[:5]
    else:
        check_tol(y2, y_ref, T, "three-launch path")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N", [1, 2, 3, 8])
def test_fused_moe_parity(fmt, N):
    log("fused moe", fmt, N)
    _check_fused(fmt, 16, 256, 64, N, 4, seed=N)


@pytest.mark.parametrize("fmt", ["int4", "nvfp4", "int5"])
@pytest.mark.parametrize("choice", [(2, 2, 2, 5, 7, 9, 11, 13), (2, 2, 2, 2, 5, 7, 9, 11)])
def test_fused_moe_shared_experts(fmt, choice):
    """Top-1 routing of eight tokens onto fewer experts, so that an output
    wave's two slots (a and a + 4) carry several routed rows: three plus one
    (int4 and NVFP4 then run both experts as the two tiles of one k-loop, the
    A operand holding four pairs) and four plus one (more than four: one
    expert after the other); int5 takes the one-at-a-time path throughout."""
    E, N = 16, 8
    rng = np.random.default_rng(sum(choice))
    logits = (0.1 * rng.standard_normal((N, E))).astype(np.float32)
    for t, e in enumerate(choice):
        logits[t, e] = 4.0
    log("fused moe shared experts", fmt, choice)
    _check_fused(fmt, E, 256, 64, N, 1, seed=0, logits=logits)


@pytest.mark.parametrize("N", [1, 2, 8])
def test_fused_moe_full_shape_int4(N):
    """The MoE workload's shapes: H = 2048, 128 experts, I = 768, top-8 routed
    on the device from seeded logits, int4 experts."""
    log("fused moe full", N)
    _check_fused("int4", 128, 2048, 768, N, 8, seed=40 + N, calls=3)


@pytest.mark.parametrize("E,H,I,N,k", [(4, 96, 32, 2, 4), (8, 160, 96, 5, 1), (3, 64, 96, 1, 3), (40, 128, 32, 8, 8),
                                       (300, 128, 32, 1, 8), (300, 96, 64, 4, 8)])
def test_fused_moe_odd_shapes(E, H, I, N, k):
    """Odd numbers of row blocks (H = 96, 160; I = 96), top_k = E (every
    expert active), top_k = 1, more selected slots than experts, and E > 256
    (the router without register-cached keys) on both paths."""
    log("fused moe ragged", E, H, I, N, k)
    _check_fused("int5", E, H, I, N, k, seed=E + H)


def test_fused_moe_no_residual_and_workspace_reuse():
    """No residual; one workspace reused across calls of different N, single
    launches (N <= 2) among them back to back: flags left by an earlier call
    never satisfy a later call's waits (each waits for its own number), and
    the flag region depends on I only, so a smaller call's data never lands
    on a larger call's flags."""
    E, H, I, k = 16, 256, 64, 4
    nbytes = qg().moe_fused_workspace_bytes(E, H, I, 8, k)
    wsp = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for N in (8, 1, 2, 1, 5):
        logits, bufs, Wgu, Wdn, xb, ids_ref, _, _ = _fused_case("nvfp4", E, H, I, N, k, seed=90 + N)
        assert qg().moe_fused_workspace_bytes(E, H, I, N, k) <= nbytes
        ys, ids, gates, w, _ = _run_fused("nvfp4", bufs, E, H, I, xb, logits, k, N, None, wsp=wsp)
        assert w[3] == 0 and np.all(w[:64] == 0), "a dependency wait timed out"
        ref_g = _ref_gates(logits, ids_ref)
        Tg = G.route_tolerance(logits, ids_ref, ref_g)
        y_ref, T = G.moe(G.x_from_bits(xb), ids_ref, ref_g, Wgu, Wdn, None, gate_tol=Tg)
        check_tol(ys[0], y_ref, T, f"fused no residual N={N}")


def test_fused_moe_rejects_bad_arguments():
    lib = qg().load()
    s = torch.cuda.current_stream().cuda_stream
    b = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = b.data_ptr()
    # missing workspace, too small workspace, top_k > E
    assert lib.qgemv_moe_fused(1, p, p, p, p, 4, 64, 32, p, p, 2, None, p, 1, None, None, None, 0, s) == -5
    assert lib.qgemv_moe_fused(1, p, p, p, p, 4, 64, 32, p, p, 2, None, p, 1, None, None, p, 16, s) == -5
    assert lib.qgemv_moe_fused(1, p, p, p, p, 4, 64, 32, p, p, 5, None, p, 1, None, None, p, 1 << 16, s) == -7
