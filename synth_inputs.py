"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random numbers
and rounds the activation-side tensors to bf16 (the compute dtype).  Both the
HIP path and the oracle read what it returns.

Recipe (every stream is numpy PCG64 seeded with base_seed + offset):
  +0 W ~ N(0, 0.02) drawn in float64 and cast to fp32 (std is the second
     argument of N(0, s));
  +1 outliers: round(0.001 * P) distinct flat indices multiplied by 10
     (only for the shapes that ask for outliers);
  +2 X ~ N(0, 1), +3 A ~ N(0, 1/r), +4 B ~ N(0, 0.01), +5 dY ~ N(0, 1),
     each drawn in float64, cast to fp32, then rounded to bf16 (RNE).
  Inside a multi-matrix workload, matrix i adds 10*i to every offset.
"""
from __future__ import annotations

import numpy as np

# Workloads, named by what they are.  c = alpha / r.
WORKLOADS = {
    "tiny_256": {"shapes": [(256, 256)], "M": 16, "r": 8, "alpha": 16.0,
                 "seed": 101, "outliers": False},
    "attn7b_4096": {"shapes": [(4096, 4096)], "M": 4096, "r": 64, "alpha": 16.0,
                    "seed": 202, "outliers": True},
    "mlp7b_4096x11008": {"shapes": [(4096, 11008), (4096, 11008), (11008, 4096)],
                         "M": 4096, "r": 16, "alpha": 32.0, "seed": 303,
                         "outliers": True},
    "decode65b_8192x22016": {"shapes": [(8192, 22016)], "M_list": [1, 8, 16],
                             "M": 16, "r": 64, "alpha": 16.0, "seed": 404,
                             "outliers": True},
    "block65b_m2048": {"shapes": [(8192, 8192)] * 4 + [(8192, 22016)] * 2 + [(22016, 8192)],
                       "M": 2048, "r": 64, "alpha": 16.0, "seed": 505,
                       "outliers": False},
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def weight(K: int, N: int, seed: int, outliers: bool, std: float = 0.02) -> np.ndarray:
    """fp32 K x N frozen weight, row-major."""
    w = (_rng(seed).standard_normal(K * N) * std).astype(np.float32)
    if outliers:
        P = K * N
        idx = _rng(seed + 1).choice(P, int(round(0.001 * P)), replace=False)
        w[idx] *= np.float32(10.0)
    return w.reshape(K, N)


def f16_normal(shape, std: float, seed: int):
    """Returns (bits uint16, values fp32) of an fp16 N(0, std) tensor (the
    fp32 draw rounded to fp16 by numpy, nearest even)."""
    n = int(np.prod(shape))
    x = (_rng(seed).standard_normal(n) * std).astype(np.float32)
    h = x.astype(np.float16).reshape(shape)
    return h.view(np.uint16), h.astype(np.float32)


def bf16_normal(shape, std: float, seed: int):
    """Returns (bits uint16, values fp32) of a bf16 N(0, std) tensor."""
    n = int(np.prod(shape))
    x = (_rng(seed).standard_normal(n) * std).astype(np.float32)
    bits = to_bf16_bits(x).reshape(shape)
    return bits, bf16_bits_to_f32(bits).reshape(shape)


def layer_inputs(name: str, matrix: int = 0, M: int | None = None,
                 with_weight: bool = True, with_grad: bool = True) -> dict:
    """All inputs of one linear of a workload (matrix index ``matrix``)."""
    wl = WORKLOADS[name]
    K, N = wl["shapes"][matrix]
    M = wl["M"] if M is None else M
    r = wl["r"]
    base = wl["seed"] + 10 * matrix
    out = {"M": M, "K": K, "N": N, "r": r, "c": wl["alpha"] / r, "name": name,
           "matrix": matrix}
    if with_weight:
        out["W"] = weight(K, N, base, wl["outliers"])
    out["X_bits"], out["X"] = bf16_normal((M, K), 1.0, base + 2)
    out["A_bits"], out["A"] = bf16_normal((K, r), 1.0 / r, base + 3)
    out["B_bits"], out["B"] = bf16_normal((r, N), 0.01, base + 4)
    if with_grad:
        out["G_bits"], out["G"] = bf16_normal((M, N), 1.0, base + 5)
    return out
