"""GPU parity of single-level states (double quantization off: one fp32 scale
per 64-block, â = absmax) against the CPU oracle, through the C ABI: the
encoder and decoder bit-exact, every layer path (dequant-GEMV, fused
dequant-GEMM, dequantize-then-GEMM) within the layer tolerance and bit-exact
on the exact-integer case, and the merge bit-exact.
"""
import numpy as np
import pytest

import bit_nf4_quantized_10_amd as qn
import synth_inputs as si
from oracle import nf4_oracle as o
from tests.gpu_util import dev_bf16, dev_f32, host, random_layer_shapes, rel_err, say
from tests.test_gpu_parity import TOL, _integer_case, _layer_case, _special_tensors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qn.lib()  # fails loudly if the HIP library is missing


def _quantize_single(w32):
    state, status = qn.nf4_quantize(dev_f32(w32), double_quant=False)
    assert not state.double_quant
    return state, qn.nf4_status_read(status)


def _assert_single_state(state, ref):
    np.testing.assert_array_equal(host(state.codes), ref["codes_packed"])
    np.testing.assert_array_equal(host(state.absmax).view(np.uint32), np.asarray(ref["absmax"]).view(np.uint32))


SPECIAL = ["P1", "P3_odd", "P65", "P16385", "tiny_zero_block", "all_zero_4096", "mixed_magnitudes", "subnormal",
           "huge_magnitudes", "midpoint_ties", "outliers_300k"]


@pytest.mark.parametrize("name", SPECIAL)
def test_single_level_quantize_dequantize_bit_exact(name):
    w = _special_tensors()[name].ravel()
    say(f"single-level quantize/dequantize: {name} P={w.size}")
    state, status = _quantize_single(w)
    assert status == 0
    ref = o.quantize(w, double_quant=False)
    _assert_single_state(state, ref)
    for dt in ("fp32", "bf16"):
        got = host(qn.nf4_dequantize(state, dt))
        np.testing.assert_array_equal(got.view(np.uint32), o.dequantize(ref, dt).view(np.uint32))


def test_single_level_flags_nonfinite():
    w = np.zeros(70000, np.float32)
    w[12345] = np.inf
    say("single-level quantize flags a non-finite weight")
    _, status = _quantize_single(w)
    assert status & qn.NF4_ENONFINITE
    _, status = _quantize_single(np.ones(70000, np.float32))
    assert status == 0


def test_single_level_full_size_bit_exact():
    W = si.weight(4096, 4096, 202, True)
    say("single-level quantize attn7b 4096x4096 full")
    state, status = _quantize_single(W)
    assert status == 0
    ref = o.quantize(W, double_quant=False)
    _assert_single_state(state, ref)
    got = host(qn.nf4_dequantize(state, "bf16"))
    np.testing.assert_array_equal(got.view(np.uint32), o.dequantize(ref, "bf16").view(np.uint32))


def _run(case, M, K, N, r):
    state, status = _quantize_single(case["W"])
    assert status == 0
    X, A, B, G = (dev_bf16(case[k]) for k in ("Xb", "Ab", "Bb", "Gb"))
    Y, Z = qn.qlora_linear_fwd(X, state, A, B, case["c"], K, N)
    dX, dA, dB = qn.qlora_linear_bwd(G, X, Z, state, A, B, case["c"], K, N)
    return Y, Z, dX, dA, dB


@pytest.mark.parametrize("M,K,N,r,c", [(16, 256, 256, 8, 2.0), (1, 512, 192, 16, 0.5), (130, 264, 320, 24, 0.25),
                                       (150, 1032, 1600, 16, 0.5), (600, 264, 320, 24, 0.5)]
                         + random_layer_shapes(6, 6464))
def test_single_level_layer_matches_oracle(M, K, N, r, c):
    say(f"single-level layer M={M} K={K} N={N} r={r}")
    case = _layer_case(M, K, N, r, c, seed=M * 3 + N)
    Y, Z, dX, dA, dB = _run(case, M, K, N, r)
    W_hat = o.dequantize(o.quantize(case["W"], double_quant=False), "bf16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], c)
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], c)
    errs = {"Y": rel_err(host(Y), Yr), "Z": rel_err(host(Z), Zr), "dX": rel_err(host(dX), dXr),
            "dA": rel_err(host(dA), dAr), "dB": rel_err(host(dB), dBr)}
    say(f"errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("M,K,N,r", [(16, 256, 256, 8), (96, 320, 384, 16), (520, 256, 320, 16)])
def test_single_level_exact_integer_case_bit_exact(M, K, N, r):
    say(f"single-level exact-integer layer M={M} K={K} N={N} r={r}")
    case = _integer_case(M, K, N, r, seed=M + N + 1)
    Y, Z, dX, dA, dB = _run(case, M, K, N, r)
    W_hat = o.dequantize(o.quantize(case["W"], double_quant=False), "bf16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], case["c"])
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], case["c"])
    for got, ref, name in ((Y, Yr, "Y"), (Z, Zr, "Z"), (dX, dXr, "dX")):
        np.testing.assert_array_equal(host(got), o.bf16_round(ref.astype(np.float32)), err_msg=name)
    np.testing.assert_array_equal(host(dA), dAr.astype(np.float32))
    np.testing.assert_array_equal(host(dB), dBr.astype(np.float32))


def test_single_level_merge_bit_exact():
    K, N, r = 130, 200, 24
    say("single-level merge bit-exact")
    rng = np.random.default_rng(4)
    W = (rng.standard_normal(K * N) * 0.02).astype(np.float32)
    state, status = _quantize_single(W)
    assert status == 0
    A = (rng.standard_normal((K, r)) / r).astype(np.float32)
    B = (rng.standard_normal((r, N)) * 0.05).astype(np.float32)
    got = host(qn.qlora_merge(state, dev_f32(A), dev_f32(B), 0.5, K, N))
    ref = o.merge(o.quantize(W, double_quant=False), A, B, 0.5, K, N).ravel()
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
