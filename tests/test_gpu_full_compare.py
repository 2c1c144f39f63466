"""Full-size layers compared with the oracle element by element, with no
sampling: every entry of Y, Z, dX, dA and dB, per output tile as well as
over the whole tensor, and the encoded state bit for bit.  Plus a direct
check of dZ = c G Bᵀ through an identity activation (page
"QLoRA：冻结的 4-bit 权重怎样参与一次微调", section "冻结权重为什么仍然需要输入梯度").

Shapes: the 7B attention projection (M = K = N = 4096, r = 64: 256 output
tiles of 256 x 256) and the 7B MLP up projection (M = 4096, K = 4096,
N = 11008, r = 16: 688 output tiles, 2.69 waves of workgroups, where the
last wave of tiles runs with part of the device idle)."""
import numpy as np
import pytest

import synth_inputs as si
from oracle import nf4_oracle as o
from tests.gpu_util import dev_bf16, host, rel_err, say

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _tile_errors(got, ref, tile=256):
    """Largest per-tile error max|got - ref| / max|ref| over all tiles of
    tile x tile (ragged at the edges), and the tile where it occurs."""
    got = np.asarray(got, np.float64)
    worst, where = 0.0, None
    for i in range(0, ref.shape[0], tile):
        for j in range(0, ref.shape[1], tile):
            e = rel_err(got[i:i + tile, j:j + tile], ref[i:i + tile, j:j + tile])
            if e > worst:
                worst, where = e, (i, j)
    return worst, where


def _run_full(name, matrix):
    import torch
    import bit_nf4_quantized_10_amd as qn
    d = si.layer_inputs(name, matrix=matrix)
    M, K, N, r, c = d["M"], d["K"], d["N"], d["r"], d["c"]
    say(f"full compare {name}[{matrix}] M={M} K={K} N={N} r={r}")
    state, status = qn.nf4_quantize(torch.from_numpy(d["W"]).cuda().reshape(-1))
    assert qn.nf4_status_read(status) == 0
    X, A, B, G = (dev_bf16(d[k]) for k in ("X_bits", "A_bits", "B_bits", "G_bits"))
    Y, Z = qn.qlora_linear_fwd(X, state, A, B, c, K, N)
    dX, dA, dB = qn.qlora_linear_bwd(G, X, Z, state, A, B, c, K, N)
    torch.cuda.synchronize()
    got = {"Y": host(Y), "Z": host(Z), "dX": host(dX), "dA": host(dA), "dB": host(dB)}
    codes, qabs, s2, off = (host(t) for t in (state.codes, state.qabsmax, state.absmax2, state.offset))
    del Y, Z, dX, dA, dB, X, A, B, G, state
    torch.cuda.empty_cache()

    st = o.quantize(d["W"])
    assert np.array_equal(codes, st["codes_packed"]), "packed codes differ"
    assert np.array_equal(qabs, st["qabsmax"]) and np.array_equal(s2, st["absmax2"])
    assert off[0] == st["offset"]
    W_hat = o.dequantize(st, "bf16").reshape(K, N)
    Yr, Zr = o.layer_forward(d["X"], W_hat, d["A"], d["B"], c)
    dXr, dAr, dBr, _ = o.layer_backward(d["G"], d["X"], W_hat, d["A"], d["B"], c)
    ref = {"Y": Yr, "Z": Zr, "dX": dXr, "dA": dAr, "dB": dBr}
    for k in ref:
        whole = rel_err(got[k], ref[k])
        tile, where = _tile_errors(got[k], ref[k])
        say(f"{k}: whole {whole:.2e}, worst 256x256 tile {tile:.2e} at {where}")
        assert whole <= TOL, (k, whole)
        assert tile <= TOL, (k, tile, where)


def test_full_compare_attn7b():
    _run_full("attn7b_4096", 0)


def test_full_compare_mlp7b_up_688_tiles():
    _run_full("mlp7b_4096x11008", 0)


@pytest.mark.parametrize("M,N", [(16, 768), (128, 1024), (512, 768), (4096, 1024)])
def test_dz_through_identity_activation(M, N):
    """With X = I (M = K; exact in bf16) the weight gradient of A is
    dA = Xᵀ dZ = dZ, so the library's dA is its own dZ, compared with the
    oracle's c G Bᵀ.  M = 16 is the small-M path, 128 the fused-decode path,
    512 and 4096 the two-pass path."""
    import torch
    import bit_nf4_quantized_10_amd as qn
    K, r, c = M, 64, 0.25
    rng = np.random.default_rng(M + N)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    Xb = si.to_bf16_bits(np.eye(M, dtype=np.float32))
    Ab, Af = si.bf16_normal((K, r), 1.0 / r, seed=M + 1)
    Bb, Bf = si.bf16_normal((r, N), 0.01, seed=M + 2)
    Gb, Gf = si.bf16_normal((M, N), 1.0, seed=M + 3)
    say(f"dZ through X = I, M = K = {M}, N = {N}")
    state, status = qn.nf4_quantize(torch.from_numpy(W).cuda().reshape(-1))
    assert qn.nf4_status_read(status) == 0
    X, A, B, G = dev_bf16(Xb), dev_bf16(Ab), dev_bf16(Bb), dev_bf16(Gb)
    _, Z = qn.qlora_linear_fwd(X, state, A, B, c, K, N)
    _, dA, _ = qn.qlora_linear_bwd(G, X, Z, state, A, B, c, K, N)
    dZr = c * (Gf.astype(np.float64) @ Bf.astype(np.float64).T)
    e = rel_err(host(dA), dZr)
    say(f"dZ error {e:.2e}")
    assert e <= TOL
    assert np.array_equal(host(Z), Af)   # Z = I A = A exactly
