"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: packed codes, second-level codes and scales, offset, dequantized
fp32/bf16 weights, and the layer outputs of the exact-integer special case.
Floating point layer outputs: max|err| / max|ref| <= 1e-2 against the fp64
oracle (the tolerance the method's target states).
"""
import hashlib

import numpy as np
import pytest

import bit_nf4_quantized_10_amd as qn
import synth_inputs as si
from oracle import nf4_oracle as o
from tests.gpu_util import OracleWeight, dev_bf16, dev_f32, host, random_layer_shapes, rel_err, say, state_to_host

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qn.lib()  # fails loudly if the HIP library is missing


def _quantize(w32):
    W = dev_f32(w32)
    state, status = qn.nf4_quantize(W)
    return state, qn.nf4_status_read(status)


def _assert_state_equal(got: dict, ref: dict):
    assert got["numel"] == ref["numel"]
    np.testing.assert_array_equal(got["codes_packed"], ref["codes_packed"])
    np.testing.assert_array_equal(got["qabsmax"], ref["qabsmax"])
    np.testing.assert_array_equal(got["absmax2"].view(np.uint32), np.asarray(ref["absmax2"]).view(np.uint32))
    assert np.float32(got["offset"]).view(np.uint32) == np.float32(ref["offset"]).view(np.uint32)


# ------------------------------------------------------------------ quantizer
def test_quantize_page_examples():
    cases = {
        "worked block": ([0.0, 0.2, -0.4, 1.0], "793f"),
        "zero block": ([0.0, 0.0], "77"),
        "merge requant": ([0.53, -0.44], "f1"),
        "layer example": ([0.5, -0.5], "f0"),
    }
    for name, (vals, hexbytes) in cases.items():
        say(f"quantize page example: {name}")
        state, status = _quantize(np.array(vals, np.float32))
        assert status == 0
        got = state_to_host(state)
        assert got["codes_packed"].tobytes().hex() == hexbytes
        _assert_state_equal(got, o.quantize(np.array(vals, np.float32)))
        rec = host(qn.nf4_dequantize(state, "fp32"))
        np.testing.assert_array_equal(rec, o.dequantize(o.quantize(np.array(vals, np.float32)), "fp32"))


def _special_tensors():
    rng = np.random.default_rng(123)
    t = {}
    t["P1"] = np.array([0.3], np.float32)
    t["P3_odd"] = np.array([0.1, -0.2, 0.05], np.float32)
    t["P65"] = (rng.standard_normal(65) * 0.02).astype(np.float32)
    t["P1000"] = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    t["P16385"] = (rng.standard_normal(16385) * 0.02).astype(np.float32)
    t["tiny_256x256"] = si.weight(256, 256, 101, False)
    z = si.weight(256, 256, 101, False).copy()
    z.ravel()[64 * 37:64 * 38] = 0.0
    t["tiny_zero_block"] = z
    t["all_zero_4096"] = np.zeros(4096, np.float32)
    mags = np.exp(rng.uniform(np.log(1e-30), np.log(1e30), 64 * 300)).astype(np.float32)
    t["mixed_magnitudes"] = (mags * np.sign(rng.standard_normal(mags.size))).astype(np.float32)
    # scales above 2^100 up to 1e38 (the reconstructed scales stay finite)
    big = np.exp(rng.uniform(np.log(1e31), np.log(1e38), 64 * 64)).astype(np.float32)
    t["huge_magnitudes"] = (big * np.sign(rng.standard_normal(big.size))).astype(np.float32)
    sub = (rng.standard_normal(64 * 40) * 1e-40).astype(np.float32)   # subnormal blocks
    t["subnormal"] = sub
    t["outliers_300k"] = si.weight(300, 1000, 7, True).ravel()
    # weights exactly on NF4 midpoints for power-of-two scales: ties -> smaller code
    C = o.NF4_CODEBOOK
    mids = (C[:-1] + C[1:]) / 2
    ties = []
    for e in range(-4, 4):
        for m in mids:
            v = np.float32(m * 2.0 ** e)
            if float(v) == m * 2.0 ** e:
                blk = np.zeros(64, np.float32)
                blk[0] = np.float32(2.0 ** e)
                blk[1] = v
                blk[2] = -v
                blk[3] = np.nextafter(v, np.float32(0))
                blk[4] = np.nextafter(v, np.float32(10))
                ties.append(blk)
    t["midpoint_ties"] = np.concatenate(ties)
    # groups with a large absmax spread: reconstructed scales may go negative
    spread = (rng.standard_normal(64 * 512) * 1e-3).astype(np.float32)
    spread[::64 * 7] = 50.0
    t["scale_spread"] = spread
    return t


@pytest.mark.parametrize("name", list(_special_tensors().keys()))
def test_quantize_dequantize_bit_exact(name):
    w = _special_tensors()[name].ravel()
    say(f"quantize/dequantize bit-exact: {name} P={w.size}")
    state, status = _quantize(w)
    assert status == 0
    ref = o.quantize(w)
    _assert_state_equal(state_to_host(state), ref)
    for dt in ("fp32", "bf16"):
        got = host(qn.nf4_dequantize(state, dt))
        exp = o.dequantize(ref, dt)
        np.testing.assert_array_equal(got.view(np.uint32), exp.view(np.uint32))


def test_quantize_flags_nonfinite():
    for bad in (np.nan, np.inf, -np.inf):
        w = np.zeros(300, np.float32)
        w[123] = bad
        say(f"quantize non-finite {bad}")
        _, status = _quantize(w)
        assert status & qn.NF4_ENONFINITE
    _, status = _quantize(np.ones(300, np.float32))
    assert status == 0


def test_dequantize_checks_pad_nibble():
    import torch
    w = np.array([0.1, -0.2, 0.05], np.float32)
    state, _ = _quantize(w)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    qn.nf4_dequantize(state, "fp32", status=status)
    assert qn.nf4_status_read(status) == 0
    state.codes[1] = (state.codes[1] & 0xF0) | 3
    qn.nf4_dequantize(state, "fp32", status=status)
    assert qn.nf4_status_read(status) & qn.NF4_EPADDING


def test_quantize_attn7b_full_bit_exact():
    W = si.weight(4096, 4096, 202, True)
    say("quantize attn7b 4096x4096 full")
    state, status = _quantize(W)
    assert status == 0
    ref = o.quantize(W)
    _assert_state_equal(state_to_host(state), ref)
    got = host(qn.nf4_dequantize(state, "bf16"))
    np.testing.assert_array_equal(got.view(np.uint32), o.dequantize(ref, "bf16").view(np.uint32))


def test_quantize_decode65b_sampled_bit_exact():
    W = si.weight(8192, 22016, 404, True)
    say("quantize decode65b 8192x22016, sampled blocks")
    state, status = _quantize(W)
    assert status == 0
    ow = OracleWeight(W)
    got = state_to_host(state)
    np.testing.assert_array_equal(got["qabsmax"], ow.q)
    np.testing.assert_array_equal(got["absmax2"].view(np.uint32), ow.s2.view(np.uint32))
    assert np.float32(got["offset"]).view(np.uint32) == np.float32(ow.offset).view(np.uint32)
    rng = np.random.default_rng(0)
    blocks = np.sort(rng.choice(ow.a.size, 4000, replace=False))
    blocks[-1] = ow.a.size - 1
    codes = ow.block_codes(blocks)
    packed = got["codes_packed"].reshape(-1, 32)[blocks]
    exp = ((codes[:, 0::2] << 4) | codes[:, 1::2]).astype(np.uint8)
    np.testing.assert_array_equal(packed, exp)
    # the decoder at this size loops over its tiles; sampled blocks of both outputs
    import torch
    idx = torch.from_numpy(blocks).cuda()
    for dt in ("fp32", "bf16"):
        full = qn.nf4_dequantize(state, dt).view(-1, 64)
        got_w = host(full[idx].contiguous().reshape(-1)).reshape(len(blocks), 64)
        del full
        np.testing.assert_array_equal(got_w, ow.weights_of_blocks(blocks, dt))


def test_quantize_largest_accepted_size_sampled_bit_exact():
    """The largest state the library accepts: 2^29 - 1 weights, an fp32 input
    just under 2 GiB (32-bit buffer offsets).  The count is odd, so the last
    block is partial (63 weights) and the last byte carries the pad code;
    its n2 = 32768 second-level groups are the most the separate offset
    kernel sums.  An all-zero block and an outlier block sit inside.  The
    second-level fields are compared in full; the codes and both
    dequantized outputs on sampled blocks, the partial last block included."""
    import torch
    P = (1 << 29) - 1
    say(f"quantize at the largest accepted size, P = {P}")
    rng = np.random.default_rng(29)
    w = rng.standard_normal(P, dtype=np.float32)
    w *= np.float32(0.02)
    zb = 4_000_001                       # an all-zero block
    w[zb * 64:(zb + 1) * 64] = 0.0
    w[(zb + 1) * 64 + 5] = np.float32(3.0)   # an outlier in the next block
    state, status = _quantize(w)
    assert status == 0
    a = o.first_level_absmax(w)
    q, s2, off = o.double_quantize(a)
    ahat = o.reconstruct_absmax(q, s2, off)
    n1 = a.size
    assert n1 == 1 << 23 and s2.size == 1 << 15
    got = state_to_host(state)
    np.testing.assert_array_equal(got["qabsmax"], q)
    np.testing.assert_array_equal(got["absmax2"].view(np.uint32), s2.view(np.uint32))
    assert np.float32(got["offset"]).view(np.uint32) == np.float32(off).view(np.uint32)
    packed = got["codes_packed"]
    assert packed.size == (P + 1) // 2
    # whole blocks: sampled, with the zero and outlier blocks
    blocks = np.unique(np.concatenate([rng.choice(n1 - 1, 3000, replace=False), [0, zb, zb + 1, n1 - 2]]))
    vals = w[: (n1 - 1) * 64].reshape(-1, 64)[blocks]
    codes = o.nf4_codes(vals.ravel(), a[blocks]).reshape(-1, 64)
    assert np.all(codes[np.searchsorted(blocks, zb)] == 7)
    exp = ((codes[:, 0::2] << 4) | codes[:, 1::2]).astype(np.uint8)
    np.testing.assert_array_equal(packed[: (n1 - 1) * 32].reshape(-1, 32)[blocks], exp)
    # the partial last block: 63 codes, then the pad code 7 in the low nibble
    tail = w[(n1 - 1) * 64:]
    assert tail.size == 63
    tcodes = o.nf4_codes(tail, a[n1 - 1:])
    texp, tlen = o.pack_nibbles(tcodes)
    assert tlen == 63 and (packed[-1] & 15) == 7
    np.testing.assert_array_equal(packed[(n1 - 1) * 32:], texp)
    # both dequantized outputs on the same blocks and the tail
    idx = torch.from_numpy((blocks[:, None] * 64 + np.arange(64)[None, :]).ravel()).cuda()
    for dt in ("fp32", "bf16"):
        full = qn.nf4_dequantize(state, dt)
        assert full.numel() == P
        got_w = host(full[idx].contiguous()).reshape(len(blocks), 64)
        got_t = host(full[(n1 - 1) * 64:].contiguous())
        del full
        exp_w = o.reconstruct_weights(codes.ravel(), np.repeat(ahat[blocks], 64), dt).reshape(-1, 64)
        exp_t = o.reconstruct_weights(tcodes, np.repeat(ahat[n1 - 1:], 63), dt)
        np.testing.assert_array_equal(got_w, exp_w)
        np.testing.assert_array_equal(got_t, exp_t)


# -------------------------------------------------------------------- layer
def _layer_case(M, K, N, r, c, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    W.ravel()[rng.choice(W.size, max(1, W.size // 1000), replace=False)] *= 10
    mk = lambda shape, std: si.bf16_normal(shape, std, int(rng.integers(1 << 30)))
    Xb, X = mk((M, K), 1.0)
    Ab, A = mk((K, r), 1.0 / r)
    Bb, B = mk((r, N), 0.01 * 10)   # a larger B makes the LoRA term visible
    Gb, G = mk((M, N), 1.0)
    return dict(W=W, Xb=Xb, X=X, Ab=Ab, A=A, Bb=Bb, B=B, Gb=Gb, G=G, c=c)


def _run_layer(case, M, K, N, r, need_dx=True):
    state, status = _quantize(case["W"])
    assert status == 0
    X, A, B, G = (dev_bf16(case[k]) for k in ("Xb", "Ab", "Bb", "Gb"))
    Y, Z = qn.qlora_linear_fwd(X, state, A, B, case["c"], K, N)
    dX, dA, dB = qn.qlora_linear_bwd(G, X, Z, state, A, B, case["c"], K, N, need_dx=need_dx)
    return state, Y, Z, dX, dA, dB


LAYER_SHAPES = [
    (16, 256, 256, 8, 2.0),      # tiny: small-M path
    (1, 64, 64, 8, 0.5),         # single row
    (8, 512, 192, 16, 1.0),
    (17, 256, 256, 8, 2.0),      # large-M path, ragged M
    (130, 264, 320, 24, 0.25),   # ragged M, K % 32 != 0, N % 128 != 0, r % 32 != 0
    (256, 512, 512, 64, 0.25),
    (600, 264, 320, 24, 0.5),    # dequantize-then-GEMM path (M >= 192), ragged everywhere
    (1024, 512, 768, 64, 0.25),  # dequantize-then-GEMM path, two row tiles x three column tiles
    (520, 64, 128, 8, 1.0),      # dense path with fewer reduction stages than LDS ring slots
    (512, 4104, 192, 16, 0.5),   # dense path, long reduction with a ragged last stage
    # reductions split across workgroups (too few output tiles for the device):
    (130, 2088, 320, 24, 0.25),  # fused forward in 7 splits, the last one ragged; dX unsplit
    (150, 1032, 1600, 16, 0.5),  # fused forward in 4 splits (ragged last), fused dX in 6
    (200, 1032, 1600, 16, 0.5),  # the same through the dense kernel (4 and 6 splits)
]


@pytest.mark.parametrize("M,K,N,r,c", LAYER_SHAPES)
def test_layer_fwd_bwd_matches_oracle(M, K, N, r, c):
    say(f"layer fwd/bwd M={M} K={K} N={N} r={r}")
    case = _layer_case(M, K, N, r, c, seed=M * 7 + K)
    state, Y, Z, dX, dA, dB = _run_layer(case, M, K, N, r)
    W_hat = o.dequantize(o.quantize(case["W"]), "bf16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], c)
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], c)
    errs = {"Y": rel_err(host(Y), Yr), "Z": rel_err(host(Z), Zr), "dX": rel_err(host(dX), dXr),
            "dA": rel_err(host(dA), dAr), "dB": rel_err(host(dB), dBr)}
    say(f"errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    # LoRA-branch isolation: Y - X Ŵ is the adapter term
    lora = host(Y).astype(np.float64) - case["X"].astype(np.float64) @ W_hat.astype(np.float64)
    assert rel_err(lora, c * Zr @ case["B"]) <= 0.1


# Small-M (dequant-GEMV) shapes at the edges of its launch: fewer rows than one
# 32-row step, K not a multiple of 32 or 64, an odd number of 128-column strips
# (the second strip of the last workgroup empty or half empty), a single strip,
# and several row-range pairs with a ragged last one.
GEMV_EDGE_SHAPES = [
    (1, 8, 64, 8, 0.5),
    (3, 72, 320, 8, 2.0),
    (16, 1000, 448, 16, 0.25),
    (5, 136, 64, 24, 1.0),
    (12, 2056, 576, 32, 0.5),
    (16, 4104, 1088, 64, 0.25),
]


@pytest.mark.parametrize("M,K,N,r,c", GEMV_EDGE_SHAPES)
def test_gemv_edge_shapes_match_oracle(M, K, N, r, c):
    say(f"dequant-GEMV edge shape M={M} K={K} N={N} r={r}")
    case = _layer_case(M, K, N, r, c, seed=M * 31 + K + N)
    state, Y, Z, dX, dA, dB = _run_layer(case, M, K, N, r)
    W_hat = o.dequantize(o.quantize(case["W"]), "bf16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], c)
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], c)
    errs = {"Y": rel_err(host(Y), Yr), "Z": rel_err(host(Z), Zr), "dX": rel_err(host(dX), dXr),
            "dA": rel_err(host(dA), dAr), "dB": rel_err(host(dB), dBr)}
    say(f"errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    # every column, including those of a half-empty last strip, is compared on its own
    col = np.abs(host(Y).astype(np.float64) - Yr).max(axis=0) / np.abs(Yr).max()
    assert col.max() <= TOL, int(col.argmax())


@pytest.mark.parametrize("M,K,N,r,c", random_layer_shapes(15, 2026))
def test_layer_random_shapes_match_oracle(M, K, N, r, c):
    say(f"layer fwd/bwd, random shape M={M} K={K} N={N} r={r}")
    case = _layer_case(M, K, N, r, c, seed=M * 13 + N)
    state, Y, Z, dX, dA, dB = _run_layer(case, M, K, N, r)
    W_hat = o.dequantize(o.quantize(case["W"]), "bf16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], c)
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], c)
    errs = {"Y": rel_err(host(Y), Yr), "Z": rel_err(host(Z), Zr), "dX": rel_err(host(dX), dXr),
            "dA": rel_err(host(dA), dAr), "dB": rel_err(host(dB), dBr)}
    say(f"errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, (k, v)


# Large-M shapes across the GEMMs' work plans: output tile counts from 6 to
# 200 (256 x 256 tiles), unsplit and split 2 to 32 ways, ragged M, K and N,
# on the fused (M < 192) and the two-pass (M >= 192) paths.  Every 256 x 256
# output tile must meet the tolerance on its own.
SPLIT_PLAN_SHAPES = [
    (192, 2048, 4096, 64, 0.25),    # forward 16 tiles in 8 splits; dX 8 tiles in 16
    (176, 4104, 1600, 16, 0.5),     # fused forward 7 tiles, ragged last stage; fused dX 17 tiles
    (448, 1032, 8192, 32, 0.5),     # forward 64 tiles in 2 splits; dX 10 tiles in 18
    (960, 264, 11008, 16, 2.0),     # forward 172 tiles unsplit; dX 8 tiles in 32 (ragged K)
    (2000, 520, 6400, 24, 0.25),    # forward 200 tiles unsplit; dX 24 tiles in 8
    (320, 8200, 768, 8, 1.0),       # forward 6 tiles in 32; dX 66 tiles in 3
    (3000, 1280, 1280, 64, 0.5),    # 60 tiles in 2 splits each way
]


@pytest.mark.parametrize("M,K,N,r,c", SPLIT_PLAN_SHAPES)
def test_layer_split_plans_match_oracle_per_tile(M, K, N, r, c):
    say(f"layer work plans M={M} K={K} N={N} r={r}")
    case = _layer_case(M, K, N, r, c, seed=M * 3 + K + N)
    state, Y, Z, dX, dA, dB = _run_layer(case, M, K, N, r)
    W_hat = o.dequantize(o.quantize(case["W"]), "bf16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], c)
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], c)
    for got, ref, name in ((Y, Yr, "Y"), (Z, Zr, "Z"), (dX, dXr, "dX"), (dA, dAr, "dA"), (dB, dBr, "dB")):
        g = host(got).astype(np.float64)
        assert rel_err(g, ref) <= TOL, (name, rel_err(g, ref))
        if name in ("Y", "dX"):
            for i in range(0, ref.shape[0], 256):
                for j in range(0, ref.shape[1], 256):
                    e = rel_err(g[i:i + 256, j:j + 256], ref[i:i + 256, j:j + 256])
                    assert e <= TOL, (name, i, j, e)


@pytest.mark.parametrize("M,K,N,r", [(192, 2048, 4096, 64), (960, 264, 11008, 16), (320, 8200, 768, 8)])
def test_layer_split_plans_exact_integer_case_bit_exact(M, K, N, r):
    say(f"layer work plans, exact-integer M={M} K={K} N={N} r={r}")
    case = _integer_case(M, K, N, r, seed=M + 7 * N)
    # sparser X and G keep the long reductions inside bf16's exact range
    rng = np.random.default_rng(M + K)
    for k in ("X", "G"):
        case[k] = case[k] * (rng.random(case[k].shape) < 0.3).astype(np.float32)
        case[k + "b"] = si.to_bf16_bits(case[k])
    state, Y, Z, dX, dA, dB = _run_layer(case, M, K, N, r)
    W_hat = o.dequantize(o.quantize(case["W"]), "bf16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], case["c"])
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], case["c"])
    for got, ref, name in ((Y, Yr, "Y"), (Z, Zr, "Z"), (dX, dXr, "dX")):
        r32 = o.bf16_round(ref.astype(np.float32))
        assert np.array_equal(r32, ref.astype(np.float32)), f"{name} not bf16-exact by construction"
        np.testing.assert_array_equal(host(got), r32, err_msg=name)
    np.testing.assert_array_equal(host(dA), dAr.astype(np.float32))
    np.testing.assert_array_equal(host(dB), dBr.astype(np.float32))


@pytest.mark.parametrize("M", [64, 256])   # fused path; two-pass path (dZ's sum then runs on its own)
def test_layer_bwd_without_dx(M):
    K, N, r = 256, 128, 16
    case = _layer_case(M, K, N, r, 0.5, seed=5)
    say(f"layer bwd with dX skipped, M={M}")
    _, _, _, dX, dA, dB = _run_layer(case, M, K, N, r, need_dx=False)
    assert dX is None
    W_hat = o.dequantize(o.quantize(case["W"]), "bf16").reshape(K, N)
    _, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], 0.5)
    assert rel_err(host(dA), dAr) <= TOL and rel_err(host(dB), dBr) <= TOL


@pytest.mark.parametrize("M", [8, 130, 600])   # dequant-GEMV, fused kernel, dequantize-then-GEMM
def test_layer_without_z(M):
    """Z is optional: a forward without Z gives the same Y, and a backward
    without Z recomputes it (for M > 16 with the forward's own kernels, so
    every output is the same bits)."""
    K, N, r, c = 512, 768, 16, 0.5
    case = _layer_case(M, K, N, r, c, seed=60 + M)
    say(f"layer without Z, M={M}")
    state, status = _quantize(case["W"])
    assert status == 0
    X, A, B, G = (dev_bf16(case[k]) for k in ("Xb", "Ab", "Bb", "Gb"))
    Y1, Z1 = qn.qlora_linear_fwd(X, state, A, B, c, K, N)
    Y2, Z2 = qn.qlora_linear_fwd(X, state, A, B, c, K, N, return_z=False)
    assert Z2 is None
    assert host(Y1).tobytes() == host(Y2).tobytes()
    g1 = qn.qlora_linear_bwd(G, X, Z1, state, A, B, c, K, N)
    g2 = qn.qlora_linear_bwd(G, X, None, state, A, B, c, K, N)
    if M > 16:
        for a, b in zip(g1, g2):
            assert host(a).tobytes() == host(b).tobytes()
    W_hat = o.dequantize(o.quantize(case["W"]), "bf16").reshape(K, N)
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], c)
    for got, ref in zip(g2, (dXr, dAr, dBr)):
        assert rel_err(host(got), ref) <= TOL


def _integer_case(M, K, N, r, seed):
    """Every block holds +-2^e, so the double quantization is exact and every
    accumulation is an exact small-integer sum in fp32 (and bf16)."""
    rng = np.random.default_rng(seed)
    e = -2
    W = rng.choice([-1.0, 0.0, 1.0], size=(K, N), p=[0.3, 0.4, 0.3]).astype(np.float32)
    W.reshape(-1, 64)[:, 0] = rng.choice([-1.0, 1.0], size=W.size // 64)
    W *= np.float32(2.0 ** e)
    sparse = lambda shape, p: rng.choice([-1.0, 0.0, 1.0], size=shape, p=[p / 2, 1 - p, p / 2]).astype(np.float32)
    X = sparse((M, K), 0.1)
    A = sparse((K, r), 0.05)
    B = sparse((r, N), 0.2)
    G = rng.integers(-2, 3, size=(M, N)).astype(np.float32) * sparse((M, N), 0.2)
    bits = lambda a: si.to_bf16_bits(a)
    return dict(W=W, X=X, A=A, B=B, G=G, Xb=bits(X), Ab=bits(A), Bb=bits(B), Gb=bits(G), c=0.5)


@pytest.mark.parametrize("M,K,N,r", [(16, 256, 256, 8), (96, 320, 384, 16), (520, 256, 320, 16),
                                     (96, 1024, 384, 16), (120, 512, 1280, 16), (300, 640, 1280, 16),
                                     (700, 1024, 512, 16),
                                     # ranks above 64: several 64-wide column chunks of Z, dZ, dA, dB
                                     (8, 256, 256, 256), (96, 320, 384, 256), (300, 640, 512, 136)])
def test_layer_exact_integer_case_bit_exact(M, K, N, r):
    say(f"exact-integer layer M={M} K={K} N={N} r={r}")
    case = _integer_case(M, K, N, r, seed=M + N)
    state, Y, Z, dX, dA, dB = _run_layer(case, M, K, N, r)
    W_hat = o.dequantize(o.quantize(case["W"]), "bf16").reshape(K, N)
    assert np.all(np.abs(W_hat) == 0.25) or np.all(np.isin(W_hat, [-0.25, 0.0, 0.25]))
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], case["c"])
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], case["c"])
    for got, ref, name in ((Y, Yr, "Y"), (Z, Zr, "Z"), (dX, dXr, "dX")):
        r32 = o.bf16_round(ref.astype(np.float32))
        assert np.array_equal(r32, ref.astype(np.float32)), f"{name} not bf16-exact by construction"
        np.testing.assert_array_equal(host(got), r32, err_msg=name)
    np.testing.assert_array_equal(host(dA), dAr.astype(np.float32))
    np.testing.assert_array_equal(host(dB), dBr.astype(np.float32))


@pytest.mark.parametrize("variant", ["W_zero", "B_zero", "c_zero"])
def test_layer_isolation_cases(variant):
    M, K, N, r = 48, 256, 192, 16
    case = _layer_case(M, K, N, r, 0.5, seed=11)
    if variant == "W_zero":
        case["W"] = np.zeros_like(case["W"])
    if variant == "B_zero":
        case["Bb"] = np.zeros_like(case["Bb"])
        case["B"] = np.zeros_like(case["B"])
    if variant == "c_zero":
        case["c"] = 0.0
    say(f"layer isolation {variant}")
    state, Y, Z, dX, dA, dB = _run_layer(case, M, K, N, r)
    W_hat = o.dequantize(o.quantize(case["W"]), "bf16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], case["c"])
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], case["c"])
    assert rel_err(host(Y), Yr) <= TOL and rel_err(host(Z), Zr) <= TOL and rel_err(host(dX), dXr) <= TOL
    if variant in ("B_zero", "c_zero"):
        assert np.all(host(dA) == 0.0)
        if variant == "c_zero":
            assert np.all(host(dB) == 0.0)
        else:
            assert rel_err(host(dB), dBr) <= TOL
    else:
        assert rel_err(host(dA), dAr) <= TOL and rel_err(host(dB), dBr) <= TOL


def test_frozen_state_unchanged_and_deterministic():
    M, K, N, r = 64, 256, 256, 16
    case = _layer_case(M, K, N, r, 1.0, seed=3)
    say("frozen state hash and determinism")
    state, status = _quantize(case["W"])
    digest = lambda: hashlib.sha256(b"".join(host(t).tobytes() for t in
                                             (state.codes, state.qabsmax, state.absmax2, state.offset))).hexdigest()
    before = digest()
    X, A, B, G = (dev_bf16(case[k]) for k in ("Xb", "Ab", "Bb", "Gb"))
    outs = []
    for _ in range(2):
        Y, Z = qn.qlora_linear_fwd(X, state, A, B, 1.0, K, N)
        dX, dA, dB = qn.qlora_linear_bwd(G, X, Z, state, A, B, 1.0, K, N)
        outs.append([host(t).tobytes() for t in (Y, Z, dX, dA, dB)])
    assert digest() == before
    assert outs[0] == outs[1]


@pytest.mark.parametrize("M", [8, 64, 600])   # dequant-GEMV, fused kernel, dequantize-then-GEMM
def test_layer_on_user_stream_sees_prior_work(M):
    """Every launch of a call goes on the caller's stream: it starts after
    work enqueued earlier there (a long product, then the overwrite of X and
    G) and finishes before later work on it.  The outputs must equal a plain
    run on the new inputs."""
    import torch
    K, N, r = 512, 768, 16
    case = _layer_case(M, K, N, r, 0.5, seed=21)
    say(f"layer on a user stream after pending work, M={M}")
    state, status = _quantize(case["W"])
    assert status == 0
    X, A, B, G = (dev_bf16(case[k]) for k in ("Xb", "Ab", "Bb", "Gb"))
    Y0, Z0 = qn.qlora_linear_fwd(X, state, A, B, 0.5, K, N)
    dX0, dA0, dB0 = qn.qlora_linear_bwd(G, X, Z0, state, A, B, 0.5, K, N)
    torch.cuda.synchronize()
    ref = [host(t).tobytes() for t in (Y0, Z0, dX0, dA0, dB0)]
    Xs, Gs = torch.zeros_like(X), torch.zeros_like(G)
    big = torch.randn(4096, 4096, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(4):
            big = big @ big * 1e-2          # keeps the stream busy for a while
        Xs.copy_(X)
        Gs.copy_(G)
        Y, Z = qn.qlora_linear_fwd(Xs, state, A, B, 0.5, K, N, stream=s)
        dX, dA, dB = qn.qlora_linear_bwd(Gs, Xs, Z, state, A, B, 0.5, K, N, stream=s)
        outs = [t.clone() for t in (Y, Z, dX, dA, dB)]
    s.synchronize()
    assert [host(t).tobytes() for t in outs] == ref


# ------------------------------------------------------- full-size workloads
def _full_size_check(name, matrix=0, M=None, row_samples=48, col_groups=3):
    d = si.layer_inputs(name, matrix=matrix, M=M)
    M, K, N, r, c = d["M"], d["K"], d["N"], d["r"], d["c"]
    say(f"full-size {name}[{matrix}] M={M} K={K} N={N} r={r}")
    state, status = _quantize(d["W"])
    assert status == 0
    X, A, B, G = (dev_bf16(d[k]) for k in ("X_bits", "A_bits", "B_bits", "G_bits"))
    Y, Z = qn.qlora_linear_fwd(X, state, A, B, c, K, N)
    dX, dA, dB = qn.qlora_linear_bwd(G, X, Z, state, A, B, c, K, N)
    ow = OracleWeight(d["W"])
    rng = np.random.default_rng(1)
    Xf, Af, Bf, Gf = (d[k].astype(np.float64) for k in ("X", "A", "B", "G"))
    Zr = Xf @ Af
    # Y on sampled 64-column groups (all rows)
    groups = rng.choice(N // 64, col_groups, replace=False)
    groups[0] = N // 64 - 1
    cols, Wc = ow.columns(groups)
    Yr = Xf @ Wc.astype(np.float64) + c * (Zr @ Bf[:, cols])
    e_y = rel_err(host(Y)[:, cols], Yr)
    # dX on sampled columns k (all rows)
    ks = rng.choice(K, row_samples, replace=False)
    ks[0] = K - 1
    dZr = c * (Gf @ Bf.T)
    dXr = Gf @ ow.rows(ks).astype(np.float64).T + dZr @ Af[ks].T
    e_dx = rel_err(host(dX)[:, ks], dXr)
    e_da = rel_err(host(dA), Xf.T @ dZr)
    e_db = rel_err(host(dB), c * (Zr.T @ Gf))
    e_z = rel_err(host(Z), Zr)
    say(f"errors Y={e_y:.2e} Z={e_z:.2e} dX={e_dx:.2e} dA={e_da:.2e} dB={e_db:.2e}")
    for v in (e_y, e_z, e_dx, e_da, e_db):
        assert v <= TOL


def test_full_size_attn7b():
    _full_size_check("attn7b_4096")


@pytest.mark.parametrize("matrix", [0, 1, 2])   # up, gate (4096 x 11008) and down (11008 x 4096)
def test_full_size_mlp7b(matrix):
    _full_size_check("mlp7b_4096x11008", matrix=matrix)


# the seven linears of a 65B block at M = 2048: q, k, v, o (8192 x 8192),
# gate, up (8192 x 22016), down (22016 x 8192)
@pytest.mark.parametrize("matrix", range(7))
def test_full_size_block65b(matrix):
    _full_size_check("block65b_m2048", matrix=matrix, row_samples=32, col_groups=2)


def test_layer_at_the_largest_accepted_operands():
    """W, Y and G each just under 2^29 elements, the per-operand limit of
    32-bit buffer offsets: K = 8192, N = 65472 (1023 blocks of 64, so the
    last column tile is partial), r = 64.  One quantized weight serves the
    three layer paths: M = 16 (dequant-GEMV), M = 130 (decode inside the
    GEMM) and M = 8192 (dequantize, then GEMM; Y and G at the limit too).
    Y and dX on sampled columns (all rows), Z, dA and dB in full."""
    import torch
    K, N, r, c = 8192, 65472, 64, 0.25
    assert K * N < 1 << 29 and 8192 * N < 1 << 29
    rng = np.random.default_rng(31)

    def bf(shape, std):
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= np.float32(std)
        bits = si.to_bf16_bits(x).reshape(shape)
        return bits, si.bf16_bits_to_f32(bits).reshape(shape)

    W = rng.standard_normal((K, N), dtype=np.float32)
    W *= np.float32(0.02)
    say(f"layer at the largest operands: quantize K={K} N={N}")
    state, status = _quantize(W)
    assert status == 0
    ow = OracleWeight(W)
    del W
    groups = np.array([0, 511, N // 64 - 1])
    ks = np.array([0, 4097, K - 1])
    cols, Wc = ow.columns(groups)
    Wr = ow.rows(ks).astype(np.float64)
    Ab, Af = bf((K, r), 1.0 / r)
    Bb, Bf = bf((r, N), 0.1)
    A, B = dev_bf16(Ab), dev_bf16(Bb)
    A64, B64 = Af.astype(np.float64), Bf.astype(np.float64)
    col_idx = torch.from_numpy(cols).cuda()
    k_idx = torch.from_numpy(ks).cuda()
    for M in (16, 130, 8192):
        say(f"layer at the largest operands M={M} K={K} N={N} r={r}")
        Xb, Xf = bf((M, K), 1.0)
        Gb, Gf = bf((M, N), 1.0)
        X, G = dev_bf16(Xb), dev_bf16(Gb)
        del Xb, Gb
        Y, Z = qn.qlora_linear_fwd(X, state, A, B, c, K, N)
        dX, dA, dB = qn.qlora_linear_bwd(G, X, Z, state, A, B, c, K, N)
        Y_s, dX_s = host(Y[:, col_idx]), host(dX[:, k_idx])
        Z_h, dA_h, dB_h = host(Z), host(dA), host(dB)
        del X, G, Y, Z, dX, dA, dB
        X64 = Xf.astype(np.float64)
        Zr = X64 @ A64
        e_y = rel_err(Y_s, X64 @ Wc.astype(np.float64) + c * (Zr @ B64[:, cols]))
        G64 = Gf.astype(np.float64)
        del Gf
        dZr = c * (G64 @ B64.T)
        e_dx = rel_err(dX_s, G64 @ Wr.T + dZr @ A64[ks].T)
        e_db = rel_err(dB_h, c * (Zr.T @ G64))
        del G64
        e_da = rel_err(dA_h, X64.T @ dZr)
        e_z = rel_err(Z_h, Zr)
        say(f"M={M} errors Y={e_y:.2e} Z={e_z:.2e} dX={e_dx:.2e} dA={e_da:.2e} dB={e_db:.2e}")
        for v in (e_y, e_z, e_dx, e_da, e_db):
            assert v <= TOL


@pytest.mark.parametrize("M", [1, 8, 16])
def test_full_size_decode65b_gemv(M):
    d = si.layer_inputs("decode65b_8192x22016", M=M, with_grad=False)
    K, N, r, c = d["K"], d["N"], d["r"], d["c"]
    say(f"decode65b GEMV M={M}")
    state, status = _quantize(d["W"])
    assert status == 0
    X, A, B = (dev_bf16(d[k]) for k in ("X_bits", "A_bits", "B_bits"))
    Y, Z = qn.qlora_linear_fwd(X, state, A, B, c, K, N)
    ow = OracleWeight(d["W"])
    groups = np.array([0, 17, 100, N // 64 - 1])
    cols, Wc = ow.columns(groups)
    Xf, Af, Bf = (d[k].astype(np.float64) for k in ("X", "A", "B"))
    Zr = Xf @ Af
    Yr = Xf @ Wc.astype(np.float64) + c * (Zr @ Bf[:, cols])
    e = rel_err(host(Y)[:, cols], Yr)
    say(f"GEMV M={M} err={e:.2e}")
    assert e <= TOL and rel_err(host(Z), Zr) <= TOL


@pytest.mark.parametrize("M", [8, 600])   # dequant-GEMV; dequantize-then-GEMM
def test_quantize_and_layer_step_in_hip_graph_replays_bit_exact(M):
    """The whole step (quantize, dequantize to bf16 and fp32, forward,
    backward) captured in one HIP graph with caller-owned buffers.  The weight
    has 2056 second-level groups, so the quantize also runs its separate
    offset kernel.  Every replay (state and outputs cleared eagerly before it)
    must reproduce the eager bytes of every output."""
    import torch
    K, N, r = 2048, 16448, 16
    rng = np.random.default_rng(90 + M)
    W = dev_f32((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    Xb, _ = si.bf16_normal((M, K), 1.0, 91)
    Ab, _ = si.bf16_normal((K, r), 1.0 / r, 92)
    Bb, _ = si.bf16_normal((r, N), 0.1, 93)
    Gb, _ = si.bf16_normal((M, N), 1.0, 94)
    X, A, B, G = dev_bf16(Xb), dev_bf16(Ab), dev_bf16(Bb), dev_bf16(Gb)
    P = K * N
    sz = qn.nf4_sizes(P)
    assert sz["n2"] > 2048
    say(f"quantize + layer step captured in a HIP graph, M={M} K={K} N={N}")
    state = qn.empty_state(P, "cuda")
    qws = torch.empty(sz["quant_workspace_bytes"], dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    fw, bw = qn.qlora_workspace_bytes(M, K, N, r)
    ws = torch.empty(max(fw, bw, 256), dtype=torch.uint8, device="cuda")
    W16 = torch.empty(P, dtype=torch.bfloat16, device="cuda")
    W32 = torch.empty(P, dtype=torch.float32, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dA = torch.empty(K, r, dtype=torch.float32, device="cuda")
    dB = torch.empty(r, N, dtype=torch.float32, device="cuda")
    outs = (state.codes, state.qabsmax, state.absmax2, state.offset, status, W16, W32, Y, Z, dX, dA, dB)

    def step():
        qn.nf4_quantize(W, state, qws, status)
        qn.nf4_dequantize(state, "bf16", out=W16, status=status)
        qn.nf4_dequantize(state, "fp32", out=W32, status=status)
        qn.qlora_linear_fwd(X, state, A, B, 0.5, K, N, Y, Z, ws)
        qn.qlora_linear_bwd(G, X, Z, state, A, B, 0.5, K, N, True, dX, dA, dB, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # eager reference (also configures the kernels)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    raw = lambda t: t.contiguous().view(torch.uint8).cpu().numpy().tobytes()
    ref = [raw(t) for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.zero_()               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [raw(t) for t in outs]
        assert got == ref, f"replay {rep}: " + ", ".join(str(i) for i, (a, b) in enumerate(zip(got, ref)) if a != b)


@pytest.mark.parametrize("M", [8, 130, 600])   # dequant-GEMV, fused kernel, dequantize-then-GEMM
def test_layer_in_hip_graph_replays_bit_exact(M):
    """Every launch of a call goes on the caller's stream and nothing is
    allocated or synchronised inside, so forward + backward can be captured
    in a HIP graph; each replay (with eager work and synchronisations in
    between) must reproduce the eager outputs bit for bit."""
    import torch
    K, N, r = 512, 768, 16
    case = _layer_case(M, K, N, r, 0.5, seed=40 + M)
    say(f"layer captured in a HIP graph, M={M}")
    state, status = _quantize(case["W"])
    assert status == 0
    X, A, B, G = (dev_bf16(case[k]) for k in ("Xb", "Ab", "Bb", "Gb"))
    fw, bw = qn.qlora_workspace_bytes(M, K, N, r)
    fws = torch.empty(max(fw, 256), dtype=torch.uint8, device="cuda")
    bws = torch.empty(max(bw, 256), dtype=torch.uint8, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dA = torch.empty(K, r, dtype=torch.float32, device="cuda")
    dB = torch.empty(r, N, dtype=torch.float32, device="cuda")

    def step():
        qn.qlora_linear_fwd(X, state, A, B, 0.5, K, N, Y, Z, fws)
        qn.qlora_linear_bwd(G, X, Z, state, A, B, 0.5, K, N, True, dX, dA, dB, bws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # eager reference (also configures the kernels)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [host(t).tobytes() for t in (Y, Z, dX, dA, dB)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (Y, Z, dX, dA, dB):
            t.zero_()               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert [host(t).tobytes() for t in (Y, Z, dX, dA, dB)] == ref, f"replay {rep}"
