"""Reference GEMV, epilogues, MoE index and combine (oracle; test infrastructure).

What the GPU path computes, written as plain definitions in fp64:
  * GEMV (NInfer article, section 2: the decode matmul over quantised
    weights, with residual add fused):
        y[n, m] = r[n, m] + sum_k x[n, k] * W[m, k]
    x is bf16 (exact in fp64), W the fp32 dequantised weights.
  * SwiGLU (same section: SwiGLU fused into the matmul): for the fused
    [2I][K] matrix, gate rows [0, I) and up rows [I, 2I):
        h[n, i] = silu(g) * u,  silu(g) = g / (1 + exp(-g))
  * MoE (Decapybara page: a top-8 softmax router; memra page: a 35B-A3B MoE
    on one card): each token t runs only its top-k experts e_j with weights
    p_j; per (t, j): h = SwiGLU(x_t W_gu[e]^T) (kept in fp64), o = h W_dn[e]^T,
    y_t = r_t + sum_j p_j o_j with j in increasing order.
  * RMSNorm prologue (same section: normalisation fused into the matmul
    that consumes it):
        x[n, k] = h[n, k] * gamma[k] / sqrt(mean_k h[n, k]^2 + eps)
    then the GEMV / SwiGLU on x.
  * MoE routing index: the (token, slot) pairs grouped by expert, ordered by
    (expert, token, slot); counts, offsets, the ascending list of active
    experts and an error flag for ids outside [0, E).
  * MX GEMV (Decapybara kernel list: an MXFP8 block-scaled GEMV fed by a
    dynamic 32-element MXFP8 activation quantiser): the activations are
    first quantised to MXFP8 (oracle.quant.mx_act_quant), then
        y[n, m] = r[n, m] + sum_k xq[n, k] * W[m, k]
    with xq the dequantised MXFP8 activations and W the dequantised MXFP8 or
    MXFP4 weights (every product is exact in fp32, so the GEMV tolerance
    below, which covers fp32 accumulation over K <= 2^17, applies as is).
  * Per-output tolerances for the fp32-accumulating GPU path:
        GEMV   T = 2e-3 * sum_k |x_k W_k| + 1e-5
        SwiGLU T_h = 1.1 (|u| + T_u) T_g + |silu(g)| T_u + 1e-6 |h| + 1e-5
               (max |silu'| < 1.1; the 1e-6 |h| term covers device exp/div)
        MoE    T_y = sum_j |p_j| (2e-3 sum_c (|h_c| + T_h,c) |Wd_c|
                                   + sum_c |Wd_c| T_h,c + 1e-5) + 1e-5
               (the down GEMV's own 2e-3 applies to the h it receives, whose
               magnitude is at most |h| + T_h)
        chain  a SwiGLU output h (bound T_h) handed to the next GEMV rounded
               to bf16: T_hb = T_h + 2^-9 (|h| + T_h), then
               T_y = 2e-3 sum_c (|h_c| + T_hb,c) |Wd_c| + sum_c T_hb,c |Wd_c| + 1e-5
"""
from __future__ import annotations

import math

import numpy as np

from . import encodings as enc

REL = 2e-3
ABS = 1e-5


def x_from_bits(x_bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [N][K] -> fp64 values."""
    return enc.f32_from_bf16_bits(x_bits).astype(np.float64)


def mx_activations(x_bits: np.ndarray) -> np.ndarray:
    """bf16 activations [N][K] -> their MXFP8 quantisation, dequantised (fp64)."""
    from .quant import MX_BLOCK, mx_act_quant
    codes, e = mx_act_quant(x_bits)
    return enc.e4m3_decode(codes) * np.repeat(enc.e8m0_decode(e), MX_BLOCK, axis=1)


def gemv(x: np.ndarray, W: np.ndarray, residual: np.ndarray | None = None) -> np.ndarray:
    """y[N][M] = residual + x[N][K] @ W[M][K]^T in fp64."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float64)
    return y


def gemv_tolerance(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    return REL * (np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(W, np.float64)).T) + ABS


def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x[n, k] = h[n, k] * gamma[k] / sqrt(mean_k h[n, k]^2 + eps), in fp64."""
    h = np.asarray(h, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    ms = np.mean(h * h, axis=1, keepdims=True)
    return h * g[None, :] / np.sqrt(ms + float(eps))


def norm_rel(K: int) -> float:
    """Relative bound (on sum_k |x_k W_k|) that a normalised GEMV adds to the
    GEMV's own 2e-3: the GPU rounds each gamma*h to bf16 once (2^-9) and
    multiplies the dot product by an fp32 norm scale (K squares summed in
    fp32, a square root and a division: under K * 2^-24 + 2^-22)."""
    return 2.0 ** -9 + K * 2.0 ** -24 + 2.0 ** -22


def norm_gemv_tolerance(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Per-output bound for y = x W^T with x = rmsnorm(...) evaluated as above."""
    K = np.asarray(x).shape[1]
    return (REL + norm_rel(K)) * (np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(W, np.float64)).T) + ABS


def swiglu_from(g, u, Tg, Tu):
    """h = silu(g) * u and its bound, from gate/up values and their bounds."""
    sg = silu(g)
    h = sg * u
    Th = 1.1 * (np.abs(u) + Tu) * Tg + np.abs(sg) * Tu + 1e-6 * np.abs(h) + ABS
    return h, Th


BF16_REL = 2.0 ** -9    # round-to-nearest-even to bfloat16


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(x: np.ndarray, W_gu: np.ndarray):
    """Fused gate/up: returns (h, T_h) for W_gu [2I][K]."""
    I = W_gu.shape[0] // 2
    g = gemv(x, W_gu[:I])
    u = gemv(x, W_gu[I:])
    Tg = gemv_tolerance(x, W_gu[:I])
    Tu = gemv_tolerance(x, W_gu[I:])
    sg = silu(g)
    h = sg * u
    Th = 1.1 * (np.abs(u) + Tu) * Tg + np.abs(sg) * Tu + 1e-6 * np.abs(h) + ABS
    return h, Th


def chain_tolerance(h: np.ndarray, Th: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """Bound for y = r + bf16(h~) . Wd^T where h~ is a GPU evaluation of h
    within Th (a SwiGLU output handed to the down projection as bf16, the
    NInfer article's chained per-format kernels, section 2). The bf16
    rounding adds at most 2^-9 |h~| <= 2^-9 (|h| + Th) to the input error;
    the down GEMV then adds its own 2e-3 bound over the inputs it actually
    sees (|h~| <= |h| + T_hb), and the input error propagates through |Wd|:
        T_hb = Th + 2^-9 (|h| + Th)
        T_y  = 2e-3 (|h| + T_hb) |Wd|^T + T_hb |Wd|^T + 1e-5
    """
    h = np.abs(np.asarray(h, np.float64))
    Th = np.asarray(Th, np.float64)
    Wa = np.abs(np.asarray(Wd, np.float64))
    Thb = Th + BF16_REL * (h + Th)
    return REL * ((h + Thb) @ Wa.T) + Thb @ Wa.T + ABS


def moe_index(ids: np.ndarray, E: int):
    """Routing index for ids [N][k] (int32).

    Returns counts[E], offsets[E+1], pairs[N*k] (flat entry t*k + j in
    (expert, token, slot) order, -1 past offsets[E]), active[E] (ascending
    experts with a nonzero count, -1 after n_active), n_active, err (1 if an
    id lies outside [0, E)).
    """
    ids = np.asarray(ids, dtype=np.int64)
    N, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.zeros(E, dtype=np.int32)
    for v in flat[valid]:
        counts[v] += 1
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    pairs = np.full(N * k, -1, dtype=np.int32)
    pos = offsets[:-1].copy()
    for idx in range(N * k):            # idx = t*k + j is already (t, j) order
        if valid[idx]:
            e = flat[idx]
            pairs[pos[e]] = idx
            pos[e] += 1
    act = np.nonzero(counts)[0].astype(np.int32)
    active = np.full(E, -1, dtype=np.int32)
    active[: act.size] = act
    err = int(not np.all(valid))
    return counts, offsets, pairs, active, int(act.size), err


def moe(x: np.ndarray, ids: np.ndarray, gates: np.ndarray, W_gu: list, W_dn: list,
        residual: np.ndarray | None = None, gate_tol: np.ndarray | None = None):
    """MoE FFN reference. x [N][H] fp64, ids/gates [N][k], W_gu[e] [2I][H],
    W_dn[e] [H][I] (fp32 dequantised). Returns (y [N][H], T_y [N][H]).
    Slots whose id is outside [0, E) contribute nothing. gate_tol [N][k]:
    a bound on how far the GPU's own mixing weights may be from `gates`
    (device routing); it adds gate_tol * |o| per slot."""
    x = np.asarray(x, dtype=np.float64)
    N, k = ids.shape
    E = len(W_gu)
    H = x.shape[1]
    y = np.zeros((N, H)) if residual is None else np.asarray(residual, np.float64).copy()
    T = np.full((N, H), ABS)
    for t in range(N):
        for j in range(k):
            e = int(ids[t, j])
            if not (0 <= e < E):
                continue
            p = float(gates[t, j])
            h, Th = swiglu(x[t: t + 1], W_gu[e])
            Wd = np.asarray(W_dn[e], np.float64)
            o = h @ Wd.T
            y[t] += p * o[0]
            To = REL * ((np.abs(h) + Th) @ np.abs(Wd).T) + Th @ np.abs(Wd).T + ABS
            T[t] += abs(p) * To[0]
            if gate_tol is not None:
                T[t] += float(gate_tol[t, j]) * (np.abs(o[0]) + To[0])
    return y, T


def route_topk_softmax(logits: np.ndarray, k: int):
    """Top-k experts per token and their mixing weights (Decapybara page,
    CUDA kernel list: a top-8 softmax router).

    Selection: largest logit first; equal logits (-0 equals +0) in increasing
    expert order; a NaN logit ranks below every number, NaNs among
    themselves in increasing order. Weights: softmax over the selected
    logits, exp(l_j - l_0) / sum_i exp(l_i - l_0), in fp64, returned as fp32.
    """
    logits = np.asarray(logits, dtype=np.float64)
    N, E = logits.shape
    ids = np.zeros((N, k), dtype=np.int32)
    gates = np.zeros((N, k), dtype=np.float32)
    for t in range(N):
        def key(e):
            v = float(logits[t, e])
            return (1, 0.0, e) if math.isnan(v) else (0, -v, e)
        order = sorted(range(E), key=key)[:k]
        sel = np.array([logits[t, e] for e in order])
        with np.errstate(invalid="ignore", over="ignore"):
            w = np.exp(sel - sel[0])
            w = w / w.sum()
        ids[t] = order
        gates[t] = w.astype(np.float32)
    return ids, gates


def route_tolerance(logits: np.ndarray, ids: np.ndarray, gates_ref: np.ndarray) -> np.ndarray:
    """Per-weight bound for an fp32 evaluation of the selected softmax
    (d_j = l_j - l_0, e_j = exp(d_j), S = sum e_j, p_j = e_j / S, each step
    rounded once, exp within 2 ulp): the relative error of p_j stays below
    2^-24 (|d_j| + 4) for e_j, 2^-24 (max|d| + 4 + k) for S and 2^-24 for the
    quotient; doubled for margin:
        T_j = p_j * 2^-23 * (|d_j| + max_i |d_i| + 9 + k) + 2^-40
    """
    logits = np.asarray(logits, np.float64)
    sel = np.take_along_axis(logits, np.asarray(ids, np.int64), 1)
    d = np.abs(sel - sel[:, :1])
    k = ids.shape[1]
    return np.asarray(gates_ref, np.float64) * 2.0 ** -23 * (d + d.max(1, keepdims=True) + 9 + k) + 2.0 ** -40


def exact_dot(xs, ws) -> "Fraction":
    """Exact sum of products of two float sequences (fractions)."""
    from fractions import Fraction
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xs, ws)), Fraction(0))


def silu_scalar(g: float) -> float:
    return g / (1.0 + math.exp(-g))
