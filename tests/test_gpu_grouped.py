"""GPU parity of grouped linears sharing X (members side by side) against the
CPU oracle applied member by member, through the C ABI."""
import numpy as np
import pytest

import bit_nf4_quantized_10_amd as qn
import synth_inputs as si
from oracle import nf4_oracle as o
from tests.gpu_util import OracleWeight, dev_bf16, dev_f32, host, rel_err, say
from tests.test_gpu_parity import TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qn.lib()  # fails loudly if the HIP library is missing


def _group_case(M, K, Ns, r, c, seed, integer=False):
    rng = np.random.default_rng(seed)
    g, Ntot = len(Ns), sum(Ns)
    if integer:
        sparse = lambda shape, p: rng.choice([-1.0, 0.0, 1.0], size=shape, p=[p / 2, 1 - p, p / 2]).astype(np.float32)
        Ws = []
        for N in Ns:
            W = rng.choice([-1.0, 0.0, 1.0], size=(K, N), p=[0.3, 0.4, 0.3]).astype(np.float32)
            W.reshape(-1, 64)[:, 0] = rng.choice([-1.0, 1.0], size=W.size // 64)
            Ws.append(W * np.float32(0.25))
        X, A, B = sparse((M, K), 0.1), sparse((K, g * r), 0.05), sparse((r, Ntot), 0.2)
        G = rng.integers(-2, 3, size=(M, Ntot)).astype(np.float32) * sparse((M, Ntot), 0.2)
        bits = si.to_bf16_bits
        return dict(Ws=Ws, X=X, A=A, B=B, G=G, Xb=bits(X), Ab=bits(A), Bb=bits(B), Gb=bits(G), c=c)
    Ws = [(rng.standard_normal((K, N)) * 0.02).astype(np.float32) for N in Ns]
    mk = lambda shape, std: si.bf16_normal(shape, std, int(rng.integers(1 << 30)))
    Xb, X = mk((M, K), 1.0)
    Ab, A = mk((K, g * r), 1.0 / r)
    Bb, B = mk((r, Ntot), 0.1)
    Gb, G = mk((M, Ntot), 1.0)
    return dict(Ws=Ws, X=X, A=A, B=B, G=G, Xb=Xb, Ab=Ab, Bb=Bb, Gb=Gb, c=c)


def _oracle(case, Ns, r, wdt="bf16"):
    """Member by member with the oracle's layer: outputs side by side, dX summed.
    wdt: the 16-bit type of the dequantized weight ("bf16" or "f16")."""
    Ys, Zs, dAs, dBs, dX = [], [], [], [], 0.0
    off = 0
    for i, N in enumerate(Ns):
        W_hat = o.dequantize(o.quantize(case["Ws"][i]), wdt).reshape(-1, N)
        A_i, B_i = case["A"][:, i * r:(i + 1) * r], case["B"][:, off:off + N]
        Y, Z = o.layer_forward(case["X"], W_hat, A_i, B_i, case["c"])
        dX_i, dA_i, dB_i, _ = o.layer_backward(case["G"][:, off:off + N], case["X"], W_hat, A_i, B_i, case["c"])
        Ys.append(Y); Zs.append(Z); dAs.append(dA_i); dBs.append(dB_i)
        dX = dX + dX_i
        off += N
    return np.hstack(Ys), np.hstack(Zs), dX, np.hstack(dAs), np.hstack(dBs)


def _dev_f16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.float16).cuda()


def _run(case, K, Ns, need_dx=True, f16=False):
    states = []
    for W in case["Ws"]:
        st, status = qn.nf4_quantize(dev_f32(W))
        assert qn.nf4_status_read(status) == 0
        states.append(st)
    dev = _dev_f16 if f16 else dev_bf16
    X, A, B, G = (dev(case[k]) for k in ("Xb", "Ab", "Bb", "Gb"))
    Y, Z = qn.qlora_grouped_fwd(X, states, A, B, case["c"], K, Ns)
    dX, dA, dB = qn.qlora_grouped_bwd(G, X, Z, states, A, B, case["c"], K, Ns, need_dx=need_dx)
    return Y, Z, dX, dA, dB


@pytest.mark.parametrize("M,K,Ns,r,c", [(600, 264, [256, 512, 256], 16, 0.5), (16, 256, [256, 256], 8, 2.0),
                                         (1000, 512, [512, 256, 768], 24, 0.25),
                                         (64, 1032, [256, 512], 16, 0.5)])   # both GEMMs split, ragged K
def test_grouped_matches_oracle(M, K, Ns, r, c):
    say(f"grouped M={M} K={K} Ns={Ns} r={r}")
    case = _group_case(M, K, Ns, r, c, seed=M + K + len(Ns))
    Y, Z, dX, dA, dB = _run(case, K, Ns)
    Yr, Zr, dXr, dAr, dBr = _oracle(case, Ns, r)
    errs = {"Y": rel_err(host(Y), Yr), "Z": rel_err(host(Z), Zr), "dX": rel_err(host(dX), dXr),
            "dA": rel_err(host(dA), dAr), "dB": rel_err(host(dB), dBr)}
    say(f"errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    # the adapter term of every member is visible on its own columns
    off = 0
    for i, N in enumerate(Ns):
        W_hat = o.dequantize(o.quantize(case["Ws"][i]), "bf16").reshape(K, N)
        lora = host(Y)[:, off:off + N].astype(np.float64) - case["X"].astype(np.float64) @ W_hat.astype(np.float64)
        assert rel_err(lora, c * Zr[:, i * r:(i + 1) * r] @ case["B"][:, off:off + N]) <= 0.1
        off += N


def _random_group_shapes(n, seed):
    """Seeded grouped shapes: 1 to 8 members of 256 to 1280 columns, ranks
    with g * r <= 256, M across the three layer paths, ragged K."""
    rng = np.random.default_rng(seed)
    bands = [(1, 17), (17, 192), (192, 900)]
    shapes = []
    for i in range(n):
        g = int(rng.choice([1, 2, 4, 5, 8]))
        lo, hi = bands[i % 3]
        r = 8 * int(rng.integers(1, 256 // (8 * g) + 1))
        Ns = [256 * int(x) for x in rng.integers(1, 6, size=g)]
        shapes.append((int(rng.integers(lo, hi)), 8 * int(rng.integers(8, 160)), Ns, r,
                       float(rng.choice([0.25, 0.5, 2.0]))))
    return shapes


@pytest.mark.parametrize("M,K,Ns,r,c", _random_group_shapes(9, 77))
def test_grouped_random_shapes_match_oracle(M, K, Ns, r, c):
    say(f"grouped, random shape M={M} K={K} Ns={Ns} r={r}")
    case = _group_case(M, K, Ns, r, c, seed=M + 3 * K)
    Y, Z, dX, dA, dB = _run(case, K, Ns)
    Yr, Zr, dXr, dAr, dBr = _oracle(case, Ns, r)
    errs = {"Y": rel_err(host(Y), Yr), "Z": rel_err(host(Z), Zr), "dX": rel_err(host(dX), dXr),
            "dA": rel_err(host(dA), dAr), "dB": rel_err(host(dB), dBr)}
    say(f"errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("M,K,Ns,r", [(96, 320, [256, 256, 512], 16), (520, 256, [256, 768], 8),
                                       # eight members: the column sums take two launches
                                       (300, 256, [256, 512, 256, 256, 768, 256, 512, 256], 24)])
def test_grouped_exact_integer_case_bit_exact(M, K, Ns, r):
    say(f"grouped exact-integer M={M} K={K} Ns={Ns} r={r}")
    case = _group_case(M, K, Ns, r, 0.5, seed=M + 3, integer=True)
    Y, Z, dX, dA, dB = _run(case, K, Ns)
    Yr, Zr, dXr, dAr, dBr = _oracle(case, Ns, r)
    for got, ref, name in ((Y, Yr, "Y"), (Z, Zr, "Z"), (dX, dXr, "dX")):
        r32 = o.bf16_round(ref.astype(np.float32))
        assert np.array_equal(r32, ref.astype(np.float32)), f"{name} not bf16-exact by construction"
        np.testing.assert_array_equal(host(got), r32, err_msg=name)
    np.testing.assert_array_equal(host(dA), dAr.astype(np.float32))
    np.testing.assert_array_equal(host(dB), dBr.astype(np.float32))


def _f16_group_case(M, K, Ns, r, c, seed):
    rng = np.random.default_rng(seed)
    g, Ntot = len(Ns), sum(Ns)
    Ws = [(rng.standard_normal((K, N)) * 0.02).astype(np.float32) for N in Ns]
    mk = lambda shape, std: si.f16_normal(shape, std, int(rng.integers(1 << 30)))
    Xb, X = mk((M, K), 1.0)
    Ab, A = mk((K, g * r), 1.0 / r)
    Bb, B = mk((r, Ntot), 0.1)
    Gb, G = mk((M, Ntot), 1.0)
    return dict(Ws=Ws, X=X, A=A, B=B, G=G, Xb=Xb, Ab=Ab, Bb=Bb, Gb=Gb, c=c)


@pytest.mark.parametrize("M,K,Ns,r,c", [(600, 264, [256, 512, 256], 16, 0.5), (16, 256, [256, 256], 8, 2.0),
                                         (64, 1032, [256, 512], 16, 0.5)] + _random_group_shapes(3, 91))
def test_grouped_f16_matches_oracle(M, K, Ns, r, c):
    """The grouped calls in the fp16 compute type (qlora_grouped_fwd_dt /
    _bwd_dt): every member against the oracle with its fp16 weight."""
    import torch
    say(f"grouped fp16 M={M} K={K} Ns={Ns} r={r}")
    case = _f16_group_case(M, K, Ns, r, c, seed=M + 7 * K + len(Ns))
    Y, Z, dX, dA, dB = _run(case, K, Ns, f16=True)
    assert Y.dtype == torch.float16 and Z.dtype == torch.float16 and dX.dtype == torch.float16
    Yr, Zr, dXr, dAr, dBr = _oracle(case, Ns, r, "f16")
    errs = {"Y": rel_err(host(Y), Yr), "Z": rel_err(host(Z), Zr), "dX": rel_err(host(dX), dXr),
            "dA": rel_err(host(dA), dAr), "dB": rel_err(host(dB), dBr)}
    say(f"errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("M,K,Ns,r", [(96, 320, [256, 256, 512], 16), (520, 256, [256, 768], 8)])
def test_grouped_f16_exact_integer_case_bit_exact(M, K, Ns, r):
    say(f"grouped fp16 exact-integer M={M} K={K} Ns={Ns} r={r}")
    case = _group_case(M, K, Ns, r, 0.5, seed=M + 11, integer=True)
    for k in ("X", "A", "B", "G"):
        case[k + "b"] = case[k].astype(np.float16).view(np.uint16)
    Y, Z, dX, dA, dB = _run(case, K, Ns, f16=True)
    Yr, Zr, dXr, dAr, dBr = _oracle(case, Ns, r, "f16")
    for got, ref, name in ((Y, Yr, "Y"), (Z, Zr, "Z"), (dX, dXr, "dX")):
        r16 = o.f16_round(ref.astype(np.float32))
        assert np.array_equal(r16, ref.astype(np.float32)), f"{name} not fp16-exact by construction"
        np.testing.assert_array_equal(host(got), r16, err_msg=name)
    np.testing.assert_array_equal(host(dA), dAr.astype(np.float32))
    np.testing.assert_array_equal(host(dB), dBr.astype(np.float32))


def test_grouped_bwd_without_dx():
    M, K, Ns, r = 64, 256, [256, 256], 8
    say("grouped bwd with dX skipped")
    case = _group_case(M, K, Ns, r, 1.0, seed=9)
    _, _, dX, dA, dB = _run(case, K, Ns, need_dx=False)
    assert dX is None
    _, _, _, dAr, dBr = _oracle(case, Ns, r)
    assert rel_err(host(dA), dAr) <= TOL and rel_err(host(dB), dBr) <= TOL


def test_grouped_full_size_qkv_7b_sampled():
    """q, k, v of the 7B attention block (K = 4096, 3 x 4096 columns, r = 64,
    M = 4096): Y and dX on sampled columns / rows, dA and dB in full."""
    import torch
    M, K, Ns, r, c = 4096, 4096, [4096, 4096, 4096], 64, 0.25
    say("grouped full size qkv 7B, sampled")
    rng = np.random.default_rng(77)
    Ws = [si.weight(K, N, 900 + i, True) for i, N in enumerate(Ns)]
    Xb, X = si.bf16_normal((M, K), 1.0, 901)
    Ab, A = si.bf16_normal((K, 3 * r), 1.0 / r, 902)
    Bb, B = si.bf16_normal((r, sum(Ns)), 0.01, 903)
    Gb, G = si.bf16_normal((M, sum(Ns)), 1.0, 904)
    case = dict(Ws=Ws, Xb=Xb, Ab=Ab, Bb=Bb, Gb=Gb, c=c)
    Y, Z, dX, dA, dB = _run(case, K, Ns)
    Xf, Af, Bf, Gf = (v.astype(np.float64) for v in (X, A, B, G))
    Zr = Xf @ Af
    assert rel_err(host(Z), Zr) <= TOL
    ows = [OracleWeight(W) for W in Ws]
    off, dXr_rows = 0, 0.0
    ks = rng.choice(K, 24, replace=False)
    ks[0] = K - 1
    dZr = c * (Gf @ np.vstack([np.hstack([Bf[:, :4096], np.zeros((r, 8192))]),
                                np.hstack([np.zeros((r, 4096)), Bf[:, 4096:8192], np.zeros((r, 4096))]),
                                np.hstack([np.zeros((r, 8192)), Bf[:, 8192:]])]).T)
    for i, N in enumerate(Ns):
        groups = rng.choice(N // 64, 2, replace=False)
        cols, Wc = ows[i].columns(groups)
        Yr = Xf @ Wc.astype(np.float64) + c * (Zr[:, i * r:(i + 1) * r] @ Bf[:, off + cols])
        assert rel_err(host(Y[:, torch.from_numpy(off + cols).cuda()]), Yr) <= TOL, i
        Wr = ows[i].rows(ks).astype(np.float64)   # Ŵ_i[ks, :]
        dXr_rows = dXr_rows + Gf[:, off:off + N] @ Wr.T
        off += N
    dXr_rows = dXr_rows + dZr @ Af[ks].T
    assert rel_err(host(dX[:, torch.from_numpy(ks).cuda()]), dXr_rows) <= TOL
    assert rel_err(host(dA), Xf.T @ dZr) <= TOL
    dBr = np.hstack([c * (Zr[:, i * r:(i + 1) * r].T @ Gf[:, 4096 * i:4096 * (i + 1)]) for i in range(3)])
    assert rel_err(host(dB), dBr) <= TOL


@pytest.mark.parametrize("M", [16, 600])
def test_grouped_in_hip_graph_replays_bit_exact(M):
    """Grouped forward + backward with caller-owned buffers captured in a HIP
    graph; each replay (outputs cleared eagerly before it) reproduces the
    eager bytes."""
    import torch
    K, Ns, r = 512, [256, 768, 512, 256, 512], 16
    say(f"grouped step captured in a HIP graph, M={M} Ns={Ns}")
    case = _group_case(M, K, Ns, r, 0.5, seed=500 + M)
    states = []
    for W in case["Ws"]:
        st, status = qn.nf4_quantize(dev_f32(W))
        assert qn.nf4_status_read(status) == 0
        states.append(st)
    X, A, B, G = (dev_bf16(case[k]) for k in ("Xb", "Ab", "Bb", "Gb"))
    g, Ntot = len(Ns), sum(Ns)
    fw, bw = qn.qlora_grouped_workspace_bytes(M, K, Ns, r)
    ws = torch.empty(max(fw, bw, 256), dtype=torch.uint8, device="cuda")
    Y = torch.empty(M, Ntot, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(M, g * r, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dA = torch.empty(K, g * r, dtype=torch.float32, device="cuda")
    dB = torch.empty(r, Ntot, dtype=torch.float32, device="cuda")
    outs = (Y, Z, dX, dA, dB)

    def step():
        qn.qlora_grouped_fwd(X, states, A, B, 0.5, K, Ns, Y, Z, ws)
        qn.qlora_grouped_bwd(G, X, Z, states, A, B, 0.5, K, Ns, True, dX, dA, dB, ws)

    raw = lambda t: t.contiguous().view(torch.uint8).cpu().numpy().tobytes()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [raw(t) for t in outs]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert [raw(t) for t in outs] == ref, f"replay {rep}"
