"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

Only random draws and the bfloat16 rounding of activations live here; none
of the quantisation, packing or GEMV arithmetic does. Every draw comes from
numpy's PCG64 (`default_rng`) with an explicit seed so that both sides of a
parity check see identical inputs.

Workloads (the shapes of the 27B-class dense layer and the 35B-A3B-style MoE
the pages run; weights and activations are random, no checkpoint is used):
  * weights  W = float32(0.02) * standard_normal  (fp32 [M][K])
  * activations x = bf16_rne(standard_normal), optionally with a fraction of
    outlier columns multiplied by 20 before rounding
  * MoE router logits standard_normal [N][E]
"""
from __future__ import annotations

import numpy as np


def rng_for(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key) if len(key) > 1 else key[0])


def weights(rng: np.random.Generator, M: int, K: int, std: float = 0.02) -> np.ndarray:
    return (np.float32(std) * rng.standard_normal((M, K), dtype=np.float32)).astype(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def activations(rng: np.random.Generator, N: int, K: int, outlier_frac: float = 0.0,
                outlier_scale: float = 20.0) -> np.ndarray:
    """bf16 bit patterns [N][K]; outlier columns (same in every row) x20."""
    a = rng.standard_normal((N, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = rng.choice(K, size=n_out, replace=False)
        a[:, cols] *= np.float32(outlier_scale)
    return bf16_bits(a)


def residual(rng: np.random.Generator, N: int, M: int) -> np.ndarray:
    return rng.standard_normal((N, M), dtype=np.float32)


def router_logits(rng: np.random.Generator, N: int, E: int) -> np.ndarray:
    return rng.standard_normal((N, E), dtype=np.float32)


def random_ids(rng: np.random.Generator, N: int, E: int, k: int) -> np.ndarray:
    """k distinct expert ids per token, uniformly drawn (a stand-in routing)."""
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(N)]).astype(np.int32)


def random_gates(rng: np.random.Generator, N: int, k: int) -> np.ndarray:
    """Positive mixing weights per token that sum to one (fp32)."""
    g = rng.random((N, k)) + 0.05
    return (g / g.sum(axis=1, keepdims=True)).astype(np.float32)


# The five workloads, by name: (M, K) shapes and formats of each matmul.
LAYER_27B = {
    "qkv": dict(M=7168, K=5120, fmt="int4"),
    "gate_up": dict(M=2 * 17408, K=5120, fmt="int5"),
    "down": dict(M=5120, K=17408, fmt="int5"),
}
MOE_35B = dict(H=2048, E=128, I=768, top_k=8)
