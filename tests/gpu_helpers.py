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
