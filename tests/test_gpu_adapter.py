"""GPU parity of the adapter operations (merge for re-export, SGD step)
against the CPU oracle, through the C ABI.

Both are bit-exact by construction: the merge accumulates exact fp64
products in a fixed order and rounds once; the SGD step is two fp32
operations and one bf16 rounding per element.
"""
import numpy as np
import pytest

import bit_nf4_quantized_10_amd as qn
import synth_inputs as si
from oracle import nf4_oracle as o
from tests.golden import floats, ints, load
from tests.gpu_util import dev_bf16, dev_f32, host, say, state_to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qn.lib()  # fails loudly if the HIP library is missing


def _quantize(w32):
    state, status = qn.nf4_quantize(dev_f32(w32))
    assert qn.nf4_status_read(status) == 0
    return state


def _adapter(K, N, r, dtype, seed):
    """A (K x r) and B (r x N) as (device tensor, host fp32 values)."""
    import torch
    rng = np.random.default_rng(seed)
    if dtype == "bf16":
        Ab, A = si.bf16_normal((K, r), 1.0 / r, int(rng.integers(1 << 30)))
        Bb, B = si.bf16_normal((r, N), 0.05, int(rng.integers(1 << 30)))
        return dev_bf16(Ab), A, dev_bf16(Bb), B
    A = (rng.standard_normal((K, r)) / r).astype(np.float32)
    B = (rng.standard_normal((r, N)) * 0.05).astype(np.float32)
    return dev_f32(A), A, dev_f32(B), B


def test_merge_page_example():
    """[P1] merge section: the worked adapter (fp32 master values) merged into
    Ŵ = [0.5, -0.5]ᵀ, then re-quantized: codes [15, 1], -0.368982, -0.207964."""
    import torch
    say("merge: page example")
    g = load("p1_merge_increment.txt")
    st = _quantize(np.array(floats(g["weight"]), np.float32))
    A = torch.tensor(floats(g["A"]), dtype=torch.float32, device="cuda").reshape(2, 1)
    B = torch.tensor(floats(g["B"]), dtype=torch.float32, device="cuda").reshape(1, 1)
    merged = host(qn.qlora_merge(st, A, B, float(g["c"]), 2, 1))
    ref = o.merge(o.quantize(np.array(floats(g["weight"]), np.float32)), host(A), host(B), float(g["c"]), 2, 1)
    np.testing.assert_array_equal(merged.view(np.uint32), ref.ravel().view(np.uint32))
    st2, status = qn.qlora_merge_requantize(st, A, B, float(g["c"]), 2, 1)
    assert qn.nf4_status_read(status) == 0
    r = load("p1_merge_requant.txt")
    codes = host(st2.codes)[0]
    assert [codes >> 4, codes & 15] == ints(r["codes"])
    rec = host(qn.nf4_dequantize(st2, "fp32"))
    tol = float(r["approx_tol"])
    assert abs(float(rec[1]) - float(r["restored_1_approx"])) < tol
    assert abs(float(np.dot(floats(r["output_x"]), rec.astype(np.float64))) - float(r["output_approx"])) < tol


@pytest.mark.parametrize("K,N,r,dtype", [(64, 128, 8, "bf16"), (130, 200, 24, "fp32"), (1, 1, 1, "fp32"),
                                         (70, 64, 40, "bf16"), (256, 320, 64, "fp32")])
def test_merge_bit_exact(K, N, r, dtype):
    """Ragged tiles (K, N not multiples of 64), r across LDS steps, both
    adapter dtypes, any N (blocks run over the flat index)."""
    say(f"merge bit-exact K={K} N={N} r={r} {dtype}")
    rng = np.random.default_rng(K * 1000 + N + r)
    W = (rng.standard_normal(K * N) * 0.02).astype(np.float32)
    st = _quantize(W)
    Ad, A, Bd, B = _adapter(K, N, r, dtype, seed=r)
    got = host(qn.qlora_merge(st, Ad, Bd, 0.5, K, N))
    ref = o.merge(o.quantize(W), A, B, 0.5, K, N).ravel()
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_merge_then_requantize_matches_oracle():
    K, N, r = 192, 256, 16
    say("merge + re-quantize state bit-exact")
    rng = np.random.default_rng(5)
    W = (rng.standard_normal(K * N) * 0.02).astype(np.float32)
    st = _quantize(W)
    Ad, A, Bd, B = _adapter(K, N, r, "bf16", seed=9)
    st2, status = qn.qlora_merge_requantize(st, Ad, Bd, 2.0, K, N)
    assert qn.nf4_status_read(status) == 0
    ref = o.quantize(o.merge(o.quantize(W), A, B, 2.0, K, N).ravel())
    got = state_to_host(st2)
    np.testing.assert_array_equal(got["codes_packed"], ref["codes_packed"])
    np.testing.assert_array_equal(got["qabsmax"], ref["qabsmax"])
    np.testing.assert_array_equal(got["absmax2"].view(np.uint32), np.asarray(ref["absmax2"]).view(np.uint32))
    assert np.float32(got["offset"]).view(np.uint32) == np.float32(ref["offset"]).view(np.uint32)


def test_merge_full_size_sampled_rows():
    """The 4096 x 4096 weight with r = 64 (the measured workload): sampled
    rows (first, last, random) bit-exact against the oracle."""
    d = si.layer_inputs("attn7b_4096", with_grad=False)
    K, N, r, c = d["K"], d["N"], d["r"], d["c"]
    say(f"merge full size K={K} N={N} r={r}, sampled rows")
    st = _quantize(d["W"])
    got = qn.qlora_merge(st, dev_bf16(d["A_bits"]), dev_bf16(d["B_bits"]), c, K, N).reshape(K, N)
    rows = np.array([0, K - 1] + list(np.random.default_rng(3).choice(K, 14, replace=False)))
    import torch
    g = host(got[torch.from_numpy(rows).cuda()])
    ref = o.merge(o.quantize(d["W"]), d["A"], d["B"], c, K, N, rows=rows)
    np.testing.assert_array_equal(g.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("masters", [False, True])
def test_sgd_step_bit_exact(masters):
    import torch
    K, N, r = 300, 192, 24
    say(f"sgd step, masters={masters}")
    rng = np.random.default_rng(17)
    Ab, A = si.bf16_normal((K, r), 1.0 / r, 1)
    Bb, B = si.bf16_normal((r, N), 0.05, 2)
    dA = (rng.standard_normal((K, r)) * 0.1).astype(np.float32)
    dB = (rng.standard_normal((r, N)) * 0.1).astype(np.float32)
    Am = (A + rng.standard_normal(A.shape).astype(np.float32) * 1e-4).astype(np.float32) if masters else None
    Bm = (B + rng.standard_normal(B.shape).astype(np.float32) * 1e-4).astype(np.float32) if masters else None
    Ad, Bd = dev_bf16(Ab), dev_bf16(Bb)
    Amd = dev_f32(Am) if masters else None
    Bmd = dev_f32(Bm) if masters else None
    qn.qlora_sgd_step(Ad, Bd, dev_f32(dA), dev_f32(dB), 0.05, Amd, Bmd)
    torch.cuda.synchronize()
    refA, refAm = o.sgd_step(A, dA, 0.05, master=Am)
    refB, refBm = o.sgd_step(B, dB, 0.05, master=Bm)
    np.testing.assert_array_equal(host(Ad).view(np.uint32), refA.view(np.uint32))
    np.testing.assert_array_equal(host(Bd).view(np.uint32), refB.view(np.uint32))
    if masters:
        np.testing.assert_array_equal(host(Amd).view(np.uint32), refAm.view(np.uint32))
        np.testing.assert_array_equal(host(Bmd).view(np.uint32), refBm.view(np.uint32))


def test_sgd_page_example_masters():
    """[P1] update of the worked adapter through fp32 masters."""
    import torch
    say("sgd: page example")
    g = load("p1_sgd_update.txt")
    a0 = np.array(floats(g["A"]), np.float32).reshape(2, 1)
    b0 = np.array(floats(g["B"]), np.float32).reshape(1, 1)
    Am, Bm = dev_f32(a0), dev_f32(b0)
    Ad = torch.zeros(2, 1, dtype=torch.bfloat16, device="cuda")
    Bd = torch.zeros(1, 1, dtype=torch.bfloat16, device="cuda")
    qn.qlora_sgd_step(Ad, Bd, dev_f32(np.array(floats(g["dA"]), np.float32).reshape(2, 1)),
                      dev_f32(np.array(floats(g["dB"]), np.float32).reshape(1, 1)),
                      float(g["learning_rate"]), Am, Bm)
    torch.cuda.synchronize()
    assert np.allclose(host(Am).ravel(), floats(g["A_updated"]), rtol=0, atol=2e-8)
    assert np.allclose(host(Bm).ravel(), floats(g["B_updated"]), rtol=0, atol=3e-8)


def test_training_step_lowers_the_loss():
    """fwd -> loss 0.5 |Y - T|^2 -> bwd with G = Y - T -> SGD on the adapter
    (fp32 masters) -> fwd: the loss falls and the frozen state is unchanged."""
    import torch
    M, K, N, r, c = 64, 256, 256, 16, 1.0
    say("one adapter training step lowers the loss")
    rng = np.random.default_rng(8)
    W = (rng.standard_normal(K * N) * 0.02).astype(np.float32)
    st = _quantize(W)
    codes_before = host(st.codes).copy()
    Xb, X = si.bf16_normal((M, K), 1.0, 31)
    Ab, A = si.bf16_normal((K, r), 1.0 / r, 32)
    Bb, B = si.bf16_normal((r, N), 0.05, 33)
    T = torch.from_numpy((rng.standard_normal((M, N)) * 0.5).astype(np.float32)).cuda()
    Xd, Ad, Bd = dev_bf16(Xb), dev_bf16(Ab), dev_bf16(Bb)
    Am, Bm = dev_f32(A), dev_f32(B)

    def loss_and_grad():
        Y, Z = qn.qlora_linear_fwd(Xd, st, Ad, Bd, c, K, N)
        diff = Y.float() - T
        return 0.5 * float((diff * diff).sum()), diff.to(torch.bfloat16).contiguous(), Z

    l0, G, Z = loss_and_grad()
    _, dA, dB = qn.qlora_linear_bwd(G, Xd, Z, st, Ad, Bd, c, K, N, need_dx=False)
    qn.qlora_sgd_step(Ad, Bd, dA, dB, 1e-3, Am, Bm)
    l1, _, _ = loss_and_grad()
    assert l1 < l0
    assert np.array_equal(host(st.codes), codes_before)


@pytest.mark.parametrize("M", [8, 300])   # dequant-GEMV; dequantize-then-GEMM
def test_training_step_in_hip_graph_replays_eager_steps(M):
    """One training step (forward, backward, SGD on the adapter through fp32
    masters, then the merge of the updated adapter) captured once in a HIP
    graph.  Replaying it three times must reproduce three eager steps bit for
    bit: the adapter changes in place, so every replay starts from the
    previous one's result."""
    import torch
    K, N, r, c, lr = 512, 384, 16, 0.5, 0.05
    say(f"training step captured in a HIP graph, M={M}")
    rng = np.random.default_rng(300 + M)
    state = _quantize((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    Xb, _ = si.bf16_normal((M, K), 1.0, 301)
    Gb, _ = si.bf16_normal((M, N), 1.0, 302)
    A0, _, B0, _ = _adapter(K, N, r, "bf16", 303)
    X, G = dev_bf16(Xb), dev_bf16(Gb)
    A, B = A0.clone(), B0.clone()
    Am, Bm = A0.float(), B0.float()
    fw, bw = qn.qlora_workspace_bytes(M, K, N, r)
    ws = torch.empty(max(fw, bw, 256), dtype=torch.uint8, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dA = torch.empty(K, r, dtype=torch.float32, device="cuda")
    dB = torch.empty(r, N, dtype=torch.float32, device="cuda")
    Wm = torch.empty(K * N, dtype=torch.float32, device="cuda")
    tracked = (Y, Z, dX, dA, dB, A, B, Am, Bm, Wm)

    def step():
        qn.qlora_linear_fwd(X, state, A, B, c, K, N, Y, Z, ws)
        qn.qlora_linear_bwd(G, X, Z, state, A, B, c, K, N, True, dX, dA, dB, ws)
        qn.qlora_sgd_step(A, B, dA, dB, lr, Am, Bm)
        qn.qlora_merge(state, A, B, c, K, N, out=Wm)

    raw = lambda t: t.contiguous().view(torch.uint8).cpu().numpy().tobytes()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    eager = []
    with torch.cuda.stream(s):
        for _ in range(3):
            step()
            s.synchronize()
            eager.append([raw(t) for t in tracked])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert eager[0] != eager[1]   # the adapter really moves
    A.copy_(A0); B.copy_(B0); Am.copy_(A0.float()); Bm.copy_(B0.float())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (Y, Z, dX, dA, dB, Wm):
            t.zero_()               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [raw(t) for t in tracked]
        assert got == eager[rep], f"replay {rep}: " + ", ".join(
            str(i) for i, (a, b) in enumerate(zip(got, eager[rep])) if a != b)
