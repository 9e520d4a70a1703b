"""Helpers for the GPU parity tests: seeded inputs, device copies, and the
oracle evaluated on exactly the bytes the GPU consumed."""
from __future__ import annotations

import numpy as np

import synthetic
from oracle import gemv as G
from oracle import layout
from oracle.dequant import dequant

FORMATS = ["int4", "int5", "int8", "nvfp4"]


def dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def oracle_weights(fmt, wq, ws, M, K):
    """fp32 [M][K] weights that the packed bytes encode (oracle unpack)."""
    return dequant(layout.unpack(fmt, M, K, wq, ws))


def tile_rows(fmt, wq, ws, M, K, rt):
    """Oracle fp32 weights of row tile rt (16 rows) read from the packed bytes."""
    _, _, RT, KS = layout.geometry(M, K)
    n = KS
    if fmt == "int8":
        q = wq[rt * n * 2048:(rt + 1) * n * 2048]
        s = ws[rt * n * 128:(rt + 1) * n * 128]
    elif fmt == "nvfp4":
        q = wq[rt * n * 1024:(rt + 1) * n * 1024]
        s = np.concatenate([ws[rt * n * 128:(rt + 1) * n * 128], ws[RT * KS * 128:]])
    else:
        q = wq[rt * n * 1024:(rt + 1) * n * 1024]
        if fmt == "int5":
            hi = RT * KS * 1024
            q = np.concatenate([q, wq[hi + rt * n * 256: hi + (rt + 1) * n * 256]])
        s = ws[rt * n * 256:(rt + 1) * n * 256]
    return oracle_weights(fmt, q, s, 16, K)


def make_case(fmt, M, K, N, seed, outliers=0.0):
    import bit_quantized_weight_amd as qg
    rng = synthetic.rng_for(7, seed, M, K)
    W = synthetic.weights(rng, M, K)
    xb = synthetic.activations(rng, N, K, outliers)
    wq, ws = qg.pack(fmt, W)
    return W, xb, wq, ws


def check_tol(y_gpu, y_ref, T, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    bad = ~(err <= T)
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} outputs outside tolerance; first {tuple(i)} "
                             f"gpu={y_gpu[tuple(i)]!r} ref={y_ref[tuple(i)]!r} tol={T[tuple(i)]!r}")
    return float((err / T).max())


def ref_gemv(fmt, wq, ws, xb, M, K, residual=None):
    W = oracle_weights(fmt, wq, ws, M, K)
    x = G.x_from_bits(xb)
    return G.gemv(x, W, residual), G.gemv_tolerance(x, W)


def moe_case(fmt, E, H, I, N, k, seed, ids=None, logits=None):
    """Expert-stacked packed weights of E experts ([2I][H] gate/up, [H][I]
    down), x, ids and gates (oracle router over seeded logits unless ids are
    given), residual, and the oracle weights of the experts in use."""
    import bit_quantized_weight_amd as qg
    rng = np.random.default_rng(seed)
    gu = [synthetic.weights(rng, 2 * I, H) for _ in range(E)]
    dn = [synthetic.weights(rng, H, I) for _ in range(E)]
    sq, ss = qg.expert_stride(fmt, 2 * I, H)
    dq, ds = qg.expert_stride(fmt, H, I)
    bufs = [np.zeros(E * sq, np.uint8), np.zeros(E * ss, np.uint8), np.zeros(E * dq, np.uint8),
            np.zeros(E * ds, np.uint8)]
    xb = synthetic.activations(rng, N, H)
    if ids is None:
        if logits is None:
            logits = synthetic.router_logits(rng, N, E)
        ids, gates = G.route_topk_softmax(logits, k)
    else:
        gates = synthetic.random_gates(rng, N, k)
    r = synthetic.residual(rng, N, H)
    used = {int(e) for e in ids.reshape(-1) if 0 <= e < E}
    Wgu, Wdn = [None] * E, [None] * E          # oracle weights of the used experts only
    for e in range(E):
        q, s = qg.pack(fmt, gu[e])
        bufs[0][e * sq: e * sq + q.size] = q
        bufs[1][e * ss: e * ss + s.size] = s
        if e in used:
            Wgu[e] = oracle_weights(fmt, q, s, 2 * I, H)
        q, s = qg.pack(fmt, dn[e])
        bufs[2][e * dq: e * dq + q.size] = q
        bufs[3][e * ds: e * ds + s.size] = s
        if e in used:
            Wdn[e] = oracle_weights(fmt, q, s, H, I)
    return bufs, Wgu, Wdn, xb, ids.astype(np.int32), gates, r
