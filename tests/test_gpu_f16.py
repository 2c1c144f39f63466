"""GPU parity of the fp16 compute type (X, A, B, G, Y, Z, dX and the
dequantized weight in fp16; fp32 accumulation) against the CPU oracle,
through the C ABI: the fp16 dequantization bit-exact, every layer path
within the layer tolerance and bit-exact on the exact-integer case, the SGD
step on fp16 parameters and the merge of fp16 adapters bit-exact."""
import numpy as np
import pytest

import bit_nf4_quantized_10_amd as qn
import synth_inputs as si
from oracle import nf4_oracle as o
from tests.gpu_util import dev_f32, host, random_layer_shapes, rel_err, say
from tests.test_gpu_parity import TOL, _integer_case, _special_tensors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qn.lib()  # fails loudly if the HIP library is missing


def dev_f16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.float16).cuda()


def _quantize(w32):
    state, status = qn.nf4_quantize(dev_f32(w32))
    assert qn.nf4_status_read(status) == 0
    return state


@pytest.mark.parametrize("name", ["P3_odd", "P16385", "tiny_zero_block", "mixed_magnitudes", "subnormal",
                                  "outliers_300k"])
def test_f16_dequantize_bit_exact(name):
    w = _special_tensors()[name].ravel()
    say(f"fp16 dequantize: {name}")
    st = _quantize(w)
    got = host(qn.nf4_dequantize(st, "f16"))
    np.testing.assert_array_equal(got.view(np.uint32), o.dequantize(o.quantize(w), "f16").view(np.uint32))


def _f16_case(M, K, N, r, c, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    mk = lambda shape, std: si.f16_normal(shape, std, int(rng.integers(1 << 30)))
    Xb, X = mk((M, K), 1.0)
    Ab, A = mk((K, r), 1.0 / r)
    Bb, B = mk((r, N), 0.1)
    Gb, G = mk((M, N), 1.0)
    return dict(W=W, X=X, A=A, B=B, G=G, Xb=Xb, Ab=Ab, Bb=Bb, Gb=Gb, c=c)


def _run(case, K, N):
    st = _quantize(case["W"])
    X, A, B, G = (dev_f16(case[k]) for k in ("Xb", "Ab", "Bb", "Gb"))
    Y, Z = qn.qlora_linear_fwd(X, st, A, B, case["c"], K, N)
    dX, dA, dB = qn.qlora_linear_bwd(G, X, Z, st, A, B, case["c"], K, N)
    import torch
    assert Y.dtype == torch.float16 and dX.dtype == torch.float16
    return Y, Z, dX, dA, dB


@pytest.mark.parametrize("M,K,N,r,c", [(16, 256, 256, 8, 2.0), (1, 512, 192, 16, 0.5), (130, 264, 320, 24, 0.25),
                                       (600, 264, 320, 24, 0.5), (1024, 512, 768, 64, 0.25),
                                       (150, 1032, 1600, 16, 0.5), (200, 1032, 1600, 16, 0.5)]
                         + random_layer_shapes(6, 1616))
def test_f16_layer_matches_oracle(M, K, N, r, c):
    say(f"fp16 layer M={M} K={K} N={N} r={r}")
    case = _f16_case(M, K, N, r, c, seed=M + 5 * N)
    Y, Z, dX, dA, dB = _run(case, K, N)
    W_hat = o.dequantize(o.quantize(case["W"]), "f16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], c)
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], c)
    errs = {"Y": rel_err(host(Y), Yr), "Z": rel_err(host(Z), Zr), "dX": rel_err(host(dX), dXr),
            "dA": rel_err(host(dA), dAr), "dB": rel_err(host(dB), dBr)}
    say(f"errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    lora = host(Y).astype(np.float64) - case["X"].astype(np.float64) @ W_hat.astype(np.float64)
    assert rel_err(lora, c * Zr @ case["B"]) <= 0.1


@pytest.mark.parametrize("M,K,N,r", [(16, 256, 256, 8), (96, 320, 384, 16), (520, 256, 320, 16)])
def test_f16_exact_integer_case_bit_exact(M, K, N, r):
    say(f"fp16 exact-integer layer M={M} K={K} N={N} r={r}")
    case = _integer_case(M, K, N, r, seed=M + N + 2)
    for k in ("X", "A", "B", "G"):
        case[k + "b"] = case[k].astype(np.float16).view(np.uint16)
    Y, Z, dX, dA, dB = _run(case, K, N)
    W_hat = o.dequantize(o.quantize(case["W"]), "f16").reshape(K, N)
    Yr, Zr = o.layer_forward(case["X"], W_hat, case["A"], case["B"], case["c"])
    dXr, dAr, dBr, _ = o.layer_backward(case["G"], case["X"], W_hat, case["A"], case["B"], case["c"])
    for got, ref, name in ((Y, Yr, "Y"), (Z, Zr, "Z"), (dX, dXr, "dX")):
        r16 = o.f16_round(ref.astype(np.float32))
        assert np.array_equal(r16, ref.astype(np.float32)), f"{name} not fp16-exact by construction"
        np.testing.assert_array_equal(host(got), r16, err_msg=name)
    np.testing.assert_array_equal(host(dA), dAr.astype(np.float32))
    np.testing.assert_array_equal(host(dB), dBr.astype(np.float32))


@pytest.mark.parametrize("masters", [False, True])
def test_f16_sgd_step_bit_exact(masters):
    import torch
    K, N, r = 300, 192, 24
    say(f"fp16 sgd step, masters={masters}")
    rng = np.random.default_rng(19)
    Ab, A = si.f16_normal((K, r), 1.0 / r, 3)
    Bb, B = si.f16_normal((r, N), 0.05, 4)
    dA = (rng.standard_normal((K, r)) * 0.1).astype(np.float32)
    dB = (rng.standard_normal((r, N)) * 0.1).astype(np.float32)
    Am = (A + rng.standard_normal(A.shape).astype(np.float32) * 1e-4).astype(np.float32) if masters else None
    Bm = (B + rng.standard_normal(B.shape).astype(np.float32) * 1e-4).astype(np.float32) if masters else None
    Ad, Bd = dev_f16(Ab), dev_f16(Bb)
    Amd = dev_f32(Am) if masters else None
    Bmd = dev_f32(Bm) if masters else None
    qn.qlora_sgd_step(Ad, Bd, dev_f32(dA), dev_f32(dB), 0.05, Amd, Bmd)
    torch.cuda.synchronize()
    refA, _ = o.sgd_step(A, dA, 0.05, master=Am, dtype="f16")
    refB, _ = o.sgd_step(B, dB, 0.05, master=Bm, dtype="f16")
    np.testing.assert_array_equal(host(Ad).view(np.uint32), refA.view(np.uint32))
    np.testing.assert_array_equal(host(Bd).view(np.uint32), refB.view(np.uint32))


def test_f16_merge_bit_exact():
    K, N, r = 130, 200, 24
    say("merge of fp16 adapters")
    rng = np.random.default_rng(6)
    W = (rng.standard_normal(K * N) * 0.02).astype(np.float32)
    st = _quantize(W)
    Ab, A = si.f16_normal((K, r), 1.0 / r, 7)
    Bb, B = si.f16_normal((r, N), 0.05, 8)
    got = host(qn.qlora_merge(st, dev_f16(Ab), dev_f16(Bb), 0.5, K, N))
    ref = o.merge(o.quantize(W), A, B, 0.5, K, N).ravel()
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
