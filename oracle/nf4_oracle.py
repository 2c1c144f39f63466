"""Oracle: a plain, slow CPU implementation of the QLoRA NF4 linear layer.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code,
table or helper with the HIP library; both sides only read the seeded inputs
made by ``synth_inputs``.

Floating point: every step runs in numpy float64 unless the method fixes an
fp32 operation (absmax, the stored scales, the reconstructed weights), in which
case numpy float32 arithmetic (one IEEE round-to-nearest-even per operation, no
fused multiply-add) is used on purpose.

Pages cited (by title and section):

[P1] "QLoRA：冻结的 4-bit 权重怎样参与一次微调" (charlestar.github.io)
     - "量化基座与可训练支路怎样相加": the layer Y = X Ŵ + c (X A) B, c = alpha/r.
     - "NF4 保存的是索引而不是均匀整数值": the 16-value codebook (7 negative, one
       exact zero, 8 positive), block absmax as a multiplier, nearest code of
       the normalised value, worked block [0, 0.2, -0.4, 1].
     - "从 NF4 索引打包成字节": the printed table values, nearest choice in
       double with ties to the smaller index, scale 1 / code 7 for an all-zero
       block, finite-input and finite-reconstruction checks, packing with the
       first code in the high nibble, code 7 as odd-length padding, the logical
       length kept beside the payload, and the checks made when unpacking.
     - "Double Quantization 压缩的是 Scale": 64-weight blocks with an fp32
       absmax, the mean of those absmax values as a global offset, the centred
       values quantized to 8 bits in blocks of 256 with one fp32 scale per
       block, decode-then-add-offset on the way back, and the storage bill.
     - "冻结权重为什么仍然需要输入梯度": dZ = c G Bᵀ, dA = Xᵀ dZ, dB = c Zᵀ G,
       dX = G Ŵᵀ + dZ Aᵀ; the packed weight has no gradient.
     - "一次完整反向与有限差分": the worked layer example (x = [1, 2], codes
       [15, 0], scale 0.5, A = [0.1, 0.2]ᵀ, B = [0.3], c = 1, target 1).
     - "Merge 后还是不是训练时的函数": re-quantizing [0.53, -0.44].
[P2] "SFT（四）：QLoRA的4-bit量化与LoRA微调原理", §6 "先理解最普通的分块量化":
     a signed absmax integer quantizer with levels [-7, 7] on [-1.2, -0.4, 0.1, 0.85];
     §21.3: double quantization is a switch that further compresses the
     first-level constants (so a state without it keeps them in fp32).
[P3] "精读笔记 · QLoRA: Efficient Finetuning of Quantized LLMs", §3.0 (store
     NF4, compute in BF16) and §3.2 (double-quantization accounting).

Readings where the pages leave a step open:
  R1  W is K x N row-major; blocks of 64 run over the flat index k*N + n.
  R2  The mean of the first-level absmax values is summed in float64 as a fixed
      tree: each group of 256 by stride-halving (pairs i, i+128, then i, i+64,
      ...; missing entries are +0), then the group sums the same way after
      padding with +0 to a power of two; offset = fl32(sum / n1).
  R3  The 8-bit second-level codebook is not printed by any page.  Reading: a
      signed linear absmax code, q in [-127, 127], value fl32(q / 127), nearest
      in double with ties to the smaller q (the P1 search rule), i.e. the P2 §6
      quantizer at 8 bits.  A group whose centred values are all zero uses
      scale 1 (the P1 zero-block convention carried over).
  R4  Reconstructed scale â = fl32(fl32(Q[q] * s2) + offset) (decode, then add
      the offset; two rounded fp32 operations, no fused multiply-add).
  R5  Reconstructed weight ŵ = fl32(C[j] * â); the compute-dtype weight is the
      round-to-nearest-even bf16 of that value.
  R6  NF4 codes are chosen with the exact first-level absmax, before the
      second level runs.

Parity status of each function (see the tests under tests/):
  nf4_codebook, first_level_absmax, nf4_codes, pack_nibbles, unpack_nibbles,
  storage_bits, layer_forward, layer_backward, bf16_round, f16_round: pinned to printed
  page values, exact rational brute force, closed forms or finite differences.
  quantize(double_quant=False) / dequantize of such a state: the codes are
  those of the double-quantized encoding (R6), and the reconstruction is
  pinned by exact rational rounding of C[j] * a and the P1 worked block.
  merge: pinned by the P1 merge example ([0.53, -0.44] -> codes [15, 1],
  -0.368982, output -0.207964) and exact special cases (c = 0, B = 0,
  power-of-two rank-1 increments).  sgd_step: pinned by the P1 update of the
  worked layer example (a, b after one step; the loss falls).
  tree_offset: pinned by exactly-summable inputs and the fsum error bound.
  reconstruct_absmax: pinned by exact rational arithmetic, both roundings of
  R4 taken on the exact values, on offsets comparable to the decoded values
  (a one-rounding or unrounded-table variant fails that pin).
  linear_absmax_table / linear_absmax_codes: pinned by the P2 §6 example,
  exact rational brute force and special cases.  The CHOICE of this codebook
  for the second level (R3) is a reading: "parity unpinned" by the pages for
  that choice, since they print no second-level table.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "NF4_CODEBOOK", "BLOCK1", "BLOCK2", "LEVELS2",
    "first_level_absmax", "nf4_codes", "pack_nibbles", "unpack_nibbles",
    "tree_offset", "linear_absmax_table", "linear_absmax_codes",
    "double_quantize", "reconstruct_absmax", "quantize", "dequantize",
    "reconstruct_weights",
    "bf16_round", "layer_forward", "layer_backward", "storage_bits",
    "counts", "merge", "sgd_step", "f16_round",
]

# [P1] "从 NF4 索引打包成字节": the sixteen reconstruction values, ascending.
# Every value is exactly representable in fp32.
NF4_CODEBOOK = np.array([
    -1.0, -0.6961928009986877, -0.5250730514526367,
    -0.39491748809814453, -0.28444138169288635, -0.18477343022823334,
    -0.09105003625154495, 0.0, 0.07958029955625534, 0.16093020141124725,
    0.24611230194568634, 0.33791524171829224, 0.44070982933044434,
    0.5626170039176941, 0.7229568362236023, 1.0,
], dtype=np.float64)

BLOCK1 = 64    # [P1] "Double Quantization 压缩的是 Scale": one absmax per 64 weights
BLOCK2 = 256   # same section: one fp32 second-level scale per 256 absmax values
LEVELS2 = 127  # reading R3: signed 8-bit linear code, q in [-127, 127]


def counts(P: int) -> tuple[int, int]:
    """n1 = ceil(P/64) first-level blocks, n2 = ceil(n1/256) second-level
    blocks ([P1] "Double Quantization 压缩的是 Scale", storage bill)."""
    n1 = -(-P // BLOCK1)
    n2 = -(-n1 // BLOCK2)
    return n1, n2


def _check_finite_nonempty(w32: np.ndarray) -> None:
    # [P1] "从 NF4 索引打包成字节": a block must be non-empty and finite.
    if w32.size == 0:
        raise ValueError("nonempty input required")
    if not np.all(np.isfinite(w32)):
        raise ValueError("finite input required")


def first_level_absmax(w32: np.ndarray) -> np.ndarray:
    """Per 64-weight block: a = max |w| (exact in fp32); an all-zero block
    takes scale 1 ([P1] "NF4 保存的是索引…", "从 NF4 索引打包成字节").
    The last block may be partial; it covers the remaining weights only."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32).ravel()
    _check_finite_nonempty(w32)
    n1, _ = counts(w32.size)
    padded = np.zeros(n1 * BLOCK1, dtype=np.float32)
    padded[: w32.size] = np.abs(w32)
    a = padded.reshape(n1, BLOCK1).max(axis=1)
    a[a == 0] = np.float32(1.0)
    return a


def _nearest(v: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest table entry to each v, distances taken in double;
    np.argmin returns the first minimum, so ties go to the smaller index
    ([P1] "从 NF4 索引打包成字节")."""
    dist = np.abs(v[:, None] - table[None, :])
    return np.argmin(dist, axis=1)


def nf4_codes(w32: np.ndarray, a32: np.ndarray, chunk: int = 1 << 18) -> np.ndarray:
    """NF4 code of each weight: nearest codebook entry to w / a, the quotient
    and the distances in double ([P1] "NF4 保存的是索引…")."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32).ravel()
    a = np.repeat(a32.astype(np.float64), BLOCK1)[: w32.size]
    out = np.empty(w32.size, dtype=np.uint8)
    for s in range(0, w32.size, chunk):
        v = w32[s:s + chunk].astype(np.float64) / a[s:s + chunk]
        out[s:s + chunk] = _nearest(v, NF4_CODEBOOK)
    return out


def pack_nibbles(codes) -> tuple[np.ndarray, int]:
    """Byte stream of a code sequence ([P1] "从 NF4 索引打包成字节"): code
    2i goes to the high nibble of byte i and code 2i+1 to its low nibble; a
    sequence of odd length gets code 7 as its last low nibble.  Returns the
    bytes and the number of codes they stand for."""
    seq = np.asarray(codes).ravel()
    n = int(seq.size)
    if n and not (0 <= int(seq.min()) and int(seq.max()) <= 15):
        raise ValueError(f"codes must lie in 0..15, got {int(seq.min())}..{int(seq.max())}")
    even = np.full(n + (n & 1), 7, dtype=np.uint8)
    even[:n] = seq
    hi, lo = even[0::2], even[1::2]
    return (hi * np.uint8(16) + lo).astype(np.uint8), n


def unpack_nibbles(payload, length: int) -> np.ndarray:
    """Code sequence of a byte stream, the inverse of pack_nibbles, with the
    two checks the page makes when reading codes back: the stream holds
    exactly ceil(length / 2) bytes, and the nibble after an odd-length
    sequence is the pad code 7 ([P1] "从 NF4 索引打包成字节")."""
    data = np.asarray(payload, dtype=np.uint8).ravel()
    need = (length + 1) // 2
    if length < 0 or data.size != need:
        raise ValueError(f"{data.size} bytes cannot hold {length} codes (expected {need})")
    if length & 1 and int(data[-1]) % 16 != 7:
        raise ValueError(f"pad nibble is {int(data[-1]) % 16}, expected 7")
    both = np.stack([data // 16, data % 16], axis=1).ravel()
    return both[:length].astype(np.uint8)


def _stride_halving(x: np.ndarray) -> np.ndarray:
    """Sum along the last axis (a power-of-two length) by repeatedly adding
    the upper half onto the lower half, in float64 (reading R2)."""
    while x.shape[-1] > 1:
        h = x.shape[-1] // 2
        x = x[..., :h] + x[..., h:]
    return x[..., 0]


def tree_offset(a32: np.ndarray) -> np.float32:
    """Global offset = mean of the first-level absmax values
    ([P1] "Double Quantization 压缩的是 Scale"), summed as reading R2."""
    a32 = np.asarray(a32, dtype=np.float32).ravel()
    n1 = a32.size
    n2 = -(-n1 // BLOCK2)
    g = np.zeros(n2 * BLOCK2, dtype=np.float64)
    g[:n1] = a32
    group_sums = _stride_halving(g.reshape(n2, BLOCK2))
    L = 1 << max(0, (n2 - 1).bit_length())
    t = np.zeros(L, dtype=np.float64)
    t[:n2] = group_sums
    total = _stride_halving(t[None, :])[0]
    return np.float32(total / np.float64(n1))


def linear_absmax_table(levels: int) -> np.ndarray:
    """Signed linear code values fl32(q / levels), q = -levels..levels
    (reading R3; P2 §6 uses levels = 7)."""
    q = np.arange(-levels, levels + 1).astype(np.float32)
    return q / np.float32(levels)


def linear_absmax_codes(values32: np.ndarray, levels: int):
    """One absmax group: s = max |v| (0 -> 1), q = nearest table entry to v / s
    in double with ties to the smaller q.  Returns (q, s)."""
    values32 = np.asarray(values32, dtype=np.float32).ravel()
    s = np.float32(np.abs(values32).max()) if values32.size else np.float32(0)
    if s == 0:
        s = np.float32(1.0)
    table = linear_absmax_table(levels).astype(np.float64)
    v = values32.astype(np.float64) / np.float64(s)
    q = _nearest(v, table).astype(np.int64) - levels
    return q, s


def double_quantize(a32: np.ndarray):
    """Second level ([P1] "Double Quantization 压缩的是 Scale", readings R2/R3):
    offset = mean(a); centred c = fl32(a - offset); per group of 256, an
    8-bit linear absmax code.  Returns (q int8[n1], s2 fp32[n2], offset fp32)."""
    a32 = np.asarray(a32, dtype=np.float32).ravel()
    offset = tree_offset(a32)
    centred = (a32 - offset).astype(np.float32)
    n1 = a32.size
    n2 = -(-n1 // BLOCK2)
    q = np.empty(n1, dtype=np.int8)
    s2 = np.empty(n2, dtype=np.float32)
    for g in range(n2):
        qg, sg = linear_absmax_codes(centred[g * BLOCK2:(g + 1) * BLOCK2], LEVELS2)
        q[g * BLOCK2:(g + 1) * BLOCK2] = qg
        s2[g] = sg
    return q, s2, offset


def reconstruct_absmax(q: np.ndarray, s2: np.ndarray, offset) -> np.ndarray:
    """â = fl32(fl32(Q[q] * s2) + offset): decode the second level, then add
    the offset back ([P1] "Double Quantization 压缩的是 Scale", reading R4)."""
    table = linear_absmax_table(LEVELS2)
    qv = table[np.asarray(q, dtype=np.int64) + LEVELS2]
    s = np.repeat(np.asarray(s2, dtype=np.float32), BLOCK2)[: qv.size]
    prod = (qv * s).astype(np.float32)
    return (prod + np.float32(offset)).astype(np.float32)


def quantize(W, double_quant: bool = True) -> dict:
    """Full encoder: flat fp32 weights -> packed NF4 codes plus double-quantized
    scales.  Also returns the intermediate first-level absmax ``a`` and the
    unpacked ``codes`` for the tests.  With double_quant=False the encoding
    stops at the first level ([P1] "Double Quantization 压缩的是 Scale": one
    fp32 absmax per 64 weights is the state; [P2] §21.3 names the switch):
    the stored scales are the exact absmax values and â = a."""
    w32 = np.ascontiguousarray(W, dtype=np.float32).ravel()
    a = first_level_absmax(w32)
    codes = nf4_codes(w32, a)
    payload, length = pack_nibbles(codes)
    if not double_quant:
        return {"numel": length, "codes_packed": payload, "absmax": a, "codes": codes,
                "double_quant": False}
    q, s2, offset = double_quantize(a)
    ahat = reconstruct_absmax(q, s2, offset)
    if not np.all(np.isfinite(ahat)):
        # [P1] "从 NF4 索引打包成字节": a non-finite reconstruction is rejected.
        raise ValueError("nonfinite reconstruction")
    return {"numel": length, "codes_packed": payload, "qabsmax": q,
            "absmax2": s2, "offset": np.float32(offset), "absmax": a,
            "codes": codes, "double_quant": True}


def bf16_round(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even, returned as float32 values (torch's
    CPU conversion is the library routine used for this step)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def f16_round(x32: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 round-to-nearest-even (values from 65520 up round to
    inf), returned as float32 values (numpy's conversion is the library
    routine used for this step); [P2] §20: the other 16-bit compute type."""
    with np.errstate(over="ignore"):   # overflow to inf is the intended result
        return np.asarray(x32, dtype=np.float32).astype(np.float16).astype(np.float32)


def dequantize(state: dict, out: str = "fp32") -> np.ndarray:
    """ŵ = fl32(C[j] * â) per weight (reading R5), optionally rounded to bf16
    (the compute dtype, [P3] §3.0).  Unpacks with the page's checks."""
    P = int(state["numel"])
    codes = unpack_nibbles(state["codes_packed"], P)
    if state.get("double_quant", True):
        ahat = reconstruct_absmax(state["qabsmax"], state["absmax2"], state["offset"])
    else:
        ahat = np.asarray(state["absmax"], dtype=np.float32)   # single level: â = a
    return reconstruct_weights(codes, np.repeat(ahat, BLOCK1)[:P], out)


def reconstruct_weights(codes, ahat_per_weight, out: str = "fp32") -> np.ndarray:
    """ŵ = fl32(C[j] * â) for each code with its block's reconstructed scale
    (reading R5), optionally rounded to bf16."""
    scale = np.asarray(ahat_per_weight, dtype=np.float32)
    w = (NF4_CODEBOOK.astype(np.float32)[np.asarray(codes, dtype=np.int64)] * scale).astype(np.float32)
    if not np.all(np.isfinite(w)):
        raise ValueError("nonfinite reconstruction")
    if out == "fp32":
        return w
    if out == "bf16":
        return bf16_round(w)
    if out == "f16":
        return f16_round(w)
    raise ValueError("out must be 'fp32', 'bf16' or 'f16'")


def layer_forward(X, W_hat, A, B, c):
    """Z = X A, Y = X Ŵ + c Z B in float64 ([P1] "量化基座与可训练支路怎样相加")."""
    X = np.asarray(X, dtype=np.float64)
    Z = X @ np.asarray(A, dtype=np.float64)
    Y = X @ np.asarray(W_hat, dtype=np.float64) + float(c) * (Z @ np.asarray(B, dtype=np.float64))
    return Y, Z


def layer_backward(G, X, W_hat, A, B, c):
    """Gradients of the layer given G = dL/dY, in float64
    ([P1] "冻结权重为什么仍然需要输入梯度"): dZ = c G Bᵀ, dA = Xᵀ dZ,
    dB = c Zᵀ G, dX = G Ŵᵀ + dZ Aᵀ.  Returns (dX, dA, dB, dZ)."""
    G = np.asarray(G, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    W_hat = np.asarray(W_hat, dtype=np.float64)
    Z = X @ A
    dZ = float(c) * (G @ B.T)
    dA = X.T @ dZ
    dB = float(c) * (Z.T @ G)
    dX = G @ W_hat.T + dZ @ A.T
    return dX, dA, dB, dZ


def merge(state: dict, A, B, c, K: int, N: int, rows=None) -> np.ndarray:
    """Merged fp32 weight for re-export ([P1] "Merge 后还是不是训练时的函数":
    the trained function is Ŵ plus the adapter, merged in high precision,
    then re-quantized as a new step).  Reading: Ŵ is the fp32 reconstruction
    (R5); the increment c A B is accumulated in float64, t = 0 .. r-1 in
    order (each product of two fp32 or bf16 values is exact in float64, one
    rounding per addition), scaled by c in float64, added to ŵ in float64
    and rounded once to fp32.  A: K x r, B: r x N (fp32 or bf16 values).
    ``rows`` (optional) restricts the result to those rows of W'."""
    w = dequantize(state, "fp32").astype(np.float64).reshape(K, N)
    A = np.asarray(A, dtype=np.float64).reshape(K, -1)
    B = np.asarray(B, dtype=np.float64).reshape(A.shape[1], N)
    if rows is not None:
        w, A = w[rows], A[rows]
    acc = np.zeros(w.shape, dtype=np.float64)
    for t in range(A.shape[1]):
        acc = acc + np.outer(A[:, t], B[t])
    return (w + np.float64(c) * acc).astype(np.float32)


def sgd_step(param, grad, lr, master=None, dtype: str = "bf16"):
    """One plain SGD update of an adapter tensor ([P1] "一次完整反向与有限差分":
    only the adapter is updated, v <- v - lr * g, and the loss must fall).
    Reading: the step is taken in fp32, p' = fl32(p - fl32(lr * g)), on the
    fp32 master copy when one is kept (else on the bf16 value read as fp32);
    the 16-bit parameter is RNE(p') in bf16 (or fp16 with dtype="f16").
    Returns (16-bit values as fp32, the new fp32 master or None)."""
    g = np.asarray(grad, dtype=np.float32)
    base = np.asarray(master if master is not None else param, dtype=np.float32)
    step = (np.float32(lr) * g).astype(np.float32)
    new = (base - step).astype(np.float32)
    rnd = f16_round if dtype == "f16" else bf16_round
    return rnd(new), (new if master is not None else None)


def storage_bits(P: int, double_quant: bool = True) -> int:
    """Bits of the stored state ([P1] "Double Quantization 压缩的是 Scale"):
    with DQ 8*ceil(P/2) + 8*n1 + 32*n2 + 32 (payload, int8 scales, fp32
    second-level scales, fp32 offset); without DQ 8*ceil(P/2) + 32*n1."""
    n1, n2 = counts(P)
    payload = 8 * ((P + 1) // 2)
    if double_quant:
        return payload + 8 * n1 + 32 * n2 + 32
    return payload + 32 * n1


if __name__ == "__main__":  # pragma: no cover - manual inspection aid
    st = quantize(np.array([0.0, 0.2, -0.4, 1.0], dtype=np.float32))
    print(st["codes"].tolist(), st["codes_packed"].tobytes().hex(), dequantize(st).tolist())
    print(math.isclose(float(dequantize(st)[1]), 0.16093020141124725))
