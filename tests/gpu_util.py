"""Helpers shared by the GPU tests: device transfer, error metrics and an
oracle view of a large weight that computes only the sampled blocks."""
from __future__ import annotations

import sys

import numpy as np

from oracle import nf4_oracle as o


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def host(t) -> np.ndarray:
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def state_to_host(state) -> dict:
    return {"numel": state.numel, "codes_packed": host(state.codes), "qabsmax": host(state.qabsmax),
            "absmax2": host(state.absmax2), "offset": np.float32(host(state.offset)[0])}


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)


class OracleWeight:
    """Oracle quantization of a K x N weight, evaluated lazily per block: the
    first-level absmax and the double quantization are computed for every
    block (cheap), NF4 codes only for the blocks a check asks for."""

    def __init__(self, W: np.ndarray):
        self.K, self.N = W.shape
        self.flat = np.ascontiguousarray(W, dtype=np.float32).ravel()
        self.a = o.first_level_absmax(self.flat)
        self.q, self.s2, self.offset = o.double_quantize(self.a)
        self.ahat = o.reconstruct_absmax(self.q, self.s2, self.offset)

    def block_codes(self, blocks: np.ndarray) -> np.ndarray:
        vals = self.flat.reshape(-1, o.BLOCK1)[blocks].ravel()
        return o.nf4_codes(vals, self.a[blocks]).reshape(len(blocks), o.BLOCK1)

    def weights_of_blocks(self, blocks: np.ndarray, out: str = "bf16") -> np.ndarray:
        codes = self.block_codes(blocks)
        return o.reconstruct_weights(codes.ravel(), np.repeat(self.ahat[blocks], o.BLOCK1), out).reshape(
            len(blocks), o.BLOCK1)

    def columns(self, groups) -> tuple[np.ndarray, np.ndarray]:
        """Ŵ[:, cols] (bf16 values) for the 64-column groups given."""
        nb = self.N // o.BLOCK1
        cols, mats = [], []
        for g in groups:
            blocks = np.arange(self.K) * nb + g
            mats.append(self.weights_of_blocks(blocks))
            cols.append(np.arange(g * 64, g * 64 + 64))
        return np.concatenate(cols), np.concatenate(mats, axis=1)

    def rows(self, ks) -> np.ndarray:
        """Ŵ[ks, :] (bf16 values)."""
        nb = self.N // o.BLOCK1
        out = []
        for k in ks:
            blocks = k * nb + np.arange(nb)
            out.append(self.weights_of_blocks(blocks).ravel())
        return np.stack(out)


def random_layer_shapes(n, seed):
    """Seeded shapes across the three layer paths (M <= 16, 17..191, >= 192),
    ragged in every dimension within the layer's rules (K % 8 == 0,
    N % 64 == 0, r % 8 == 0, r <= 256)."""
    rng = np.random.default_rng(seed)
    bands = [(1, 17), (17, 192), (192, 1300)]
    shapes = []
    for i in range(n):
        lo, hi = bands[i % 3]
        shapes.append((int(rng.integers(lo, hi)), 8 * int(rng.integers(8, 200)), 64 * int(rng.integers(1, 26)),
                       8 * int(rng.integers(1, 33)), float(rng.choice([0.25, 0.5, 2.0]))))
    return shapes
