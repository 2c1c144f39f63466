"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each check compares the oracle with something other than itself: values the
pages print (tests/golden/), exact rational arithmetic (fractions.Fraction),
closed forms, finite differences and special cases.  CPU only.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4_oracle as o
from tests.golden import floats, ints, load

NF4 = [Fraction(float(v)) for v in o.NF4_CODEBOOK]


# ----------------------------------------------------------------- exact helpers
def exact_nearest(v: Fraction, table) -> int:
    """Nearest entry in exact rational arithmetic, ties to the smaller index."""
    return min(range(len(table)), key=lambda j: (abs(v - table[j]), j))


def exact_round_f32(x: Fraction) -> np.float32:
    """Round a rational to the nearest fp32, ties to even (normal range)."""
    f = np.float32(float(x))
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def exact_round_bf16(x: float) -> float:
    """Round an fp32 value to bf16, nearest with ties to even, via rationals."""
    u = int(np.array(x, np.float32).view(np.uint32))
    lo = np.array(u & 0xFFFF0000, np.uint32).view(np.float32)
    hi = np.array((u & 0xFFFF0000) + 0x10000, np.uint32).view(np.float32)
    fx = Fraction(float(x))
    dl, dh = abs(fx - Fraction(float(lo))), abs(Fraction(float(hi)) - fx)
    if dl < dh:
        return float(lo)
    if dh < dl:
        return float(hi)
    return float(lo) if ((u >> 16) & 1) == 0 else float(hi)


# --------------------------------------------------------------------- codebook
def test_codebook_invariants():
    C = o.NF4_CODEBOOK
    assert C.size == 16
    assert np.all(np.diff(C) > 0)
    assert C[0] == -1.0 and C[7] == 0.0 and C[15] == 1.0
    assert int((C < 0).sum()) == 7 and int((C > 0).sum()) == 8
    # every printed value is an exact fp32 number
    assert np.all(C.astype(np.float32).astype(np.float64) == C)


# ------------------------------------------------------------ page examples (P1)
def test_worked_block():
    g = load("p1_worked_block.txt")
    w = np.array(floats(g["input"]), np.float32)
    st = o.quantize(w)
    assert st["absmax"].tolist() == floats(g["absmax"])
    assert st["codes"].tolist() == ints(g["codes"])
    assert st["codes_packed"].tobytes().hex() == g["payload_hex"]
    assert o.unpack_nibbles(st["codes_packed"], st["numel"]).tolist() == ints(g["codes"])
    # one block => the second level reproduces the absmax exactly
    rec = o.dequantize(st, "fp32")
    assert rec.astype(np.float64).tolist() == floats(g["restored"])


def test_zero_block_and_odd_roundtrip():
    g = load("p1_zero_and_odd.txt")
    st = o.quantize(np.array(floats(g["zero_input"]), np.float32))
    assert st["codes"].tolist() == ints(g["zero_codes"])
    assert st["absmax"].tolist() == [float(g["zero_scale"])]
    assert o.dequantize(st).tolist() == [0.0, 0.0]
    payload, length = o.pack_nibbles(ints(g["odd_codes"]))
    assert payload.tobytes().hex() == g["odd_payload_hex"] and length == int(g["odd_length"])
    assert o.unpack_nibbles(payload, length).tolist() == ints(g["odd_codes"])


def test_unpack_rejects_bad_length_and_padding():
    payload, length = o.pack_nibbles([7, 15, 0])
    with pytest.raises(ValueError):
        o.unpack_nibbles(payload, 5)
    bad = payload.copy()
    bad[-1] = (bad[-1] & 0xF0) | 3
    with pytest.raises(ValueError):
        o.unpack_nibbles(bad, 3)
    with pytest.raises(ValueError):
        o.pack_nibbles([16])


def test_rejects_nonfinite_and_empty():
    for bad in ([1.0, np.nan], [np.inf, 0.0], []):
        with pytest.raises(ValueError):
            o.quantize(np.array(bad, np.float32))


def test_merge_requantize_example():
    g = load("p1_merge_requant.txt")
    st = o.quantize(np.array(floats(g["input"]), np.float32))
    assert st["codes"].tolist() == ints(g["codes"])
    rec = o.dequantize(st, "fp32")
    tol = float(g["approx_tol"])
    assert rec[1] != np.float32(-0.44)
    assert abs(float(rec[1]) - float(g["restored_1_approx"])) < tol
    y = float(np.dot(np.array(floats(g["output_x"])), rec.astype(np.float64)))
    assert abs(y - float(g["output_approx"])) < tol


def exact_round_f16(x: float) -> float:
    """Round a value to fp16, nearest with ties to even, by exact rationals
    over the fp16 grid (subnormal spacing 2^-24; 65520 and up -> inf)."""
    fx = Fraction(float(x))
    if abs(fx) >= 65520:
        return math.copysign(math.inf, float(x))
    e = max(math.floor(math.log2(abs(fx))) if fx != 0 else -24, -14)
    q = Fraction(2) ** (e - 10)            # spacing of the binade (or of subnormals)
    k = fx / q
    lo = math.floor(k)
    rem = k - lo
    n = lo + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else lo
    return float(n * q)


def test_f16_round_exact():
    vals = [1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -24 * 1.5, 2.0 ** -25, 2.0 ** -26, 65504.0, 65519.99,
            65520.0, -65536.0, 0.1, -0.16093020141124725, 3.0e-6, 1.0 / 3.0, 1234.567]
    rng = np.random.default_rng(5)
    vals += list((rng.standard_normal(300) * 10.0 ** rng.uniform(-7, 4.8, 300)).astype(np.float32))
    got = o.f16_round(np.array(vals, np.float32))
    for v, g in zip(vals, got):
        assert float(g) == exact_round_f16(float(np.float32(v))), v


def test_single_level_state():
    """Double quantization off: the codes are those of the double-quantized
    encoding (they use the exact absmax either way), the stored scales are
    the exact block maxima, and each weight is the exactly rounded fp32 of
    C[j] * a; the page's worked block reconstructs to the printed values."""
    st = o.quantize(np.array([0.0, 0.2, -0.4, 1.0], np.float32), double_quant=False)
    assert st["codes"].tolist() == [7, 9, 3, 15] and st["codes_packed"].tobytes().hex() == "793f"
    assert o.dequantize(st, "fp32").tolist() == [0.0, 0.16093020141124725, -0.39491748809814453, 1.0]
    rng = np.random.default_rng(21)
    w = (rng.standard_normal(64 * 9 + 17) * np.repeat(10.0 ** rng.uniform(-6, 6, 10), 64)[:64 * 9 + 17]).astype(np.float32)
    single, dq = o.quantize(w, double_quant=False), o.quantize(w)
    assert np.array_equal(single["codes"], dq["codes"])
    for b in range(single["absmax"].size):
        blk = w[64 * b: 64 * b + 64]
        assert single["absmax"][b] == (np.max(np.abs(blk)) or np.float32(1.0))
    rec = o.dequantize(single, "fp32")
    for i in range(w.size):
        want = exact_round_f32(NF4[int(single["codes"][i])] * Fraction(float(single["absmax"][i // 64])))
        assert rec[i] == want
    assert o.storage_bits(64 * 1024, double_quant=False) / (64 * 1024) == 4.5


def test_merge_page_example():
    """The merge of the worked adapter: increment [0.03, 0.06], merged
    [0.53, -0.44] (within the fp32 rounding of the fp32 adapter values), the
    output still -0.35; re-quantized: codes [15, 1], -0.368982, -0.207964."""
    g = load("p1_merge_increment.txt")
    st = o.quantize(np.array(floats(g["weight"]), np.float32))
    A = np.array(floats(g["A"]), np.float32).reshape(2, 1)
    B = np.array(floats(g["B"]), np.float32).reshape(1, 1)
    merged = o.merge(st, A, B, float(g["c"]), 2, 1).ravel()
    for got, want in zip(merged, floats(g["merged"])):
        w32 = np.float32(want)
        assert abs(float(got) - float(w32)) <= abs(float(np.spacing(w32)))   # one fp32 ulp
    inc = merged.astype(np.float64) - o.dequantize(st, "fp32").astype(np.float64)
    assert np.allclose(inc, floats(g["increment"]), rtol=0, atol=1e-7)
    y = float(np.dot(floats(g["x"]), merged.astype(np.float64)))
    assert abs(y - float(g["merged_output"])) < 1e-7
    r = load("p1_merge_requant.txt")
    st2 = o.quantize(merged)
    assert st2["codes"].tolist() == ints(r["codes"])
    rec = o.dequantize(st2, "fp32")
    tol = float(r["approx_tol"])
    assert abs(float(rec[1]) - float(r["restored_1_approx"])) < tol
    y2 = float(np.dot(floats(r["output_x"]), rec.astype(np.float64)))
    assert abs(y2 - float(r["output_approx"])) < tol


def test_merge_exact_rational_and_special_cases():
    """With values whose float64 sums are exact (small integers times powers
    of two), merge must equal the exactly rounded fp32 of ŵ + c Σ_t A B; with
    c = 0 or B = 0 it must return Ŵ (not W)."""
    rng = np.random.default_rng(11)
    K, N, r = 3, 64, 5
    W = (rng.standard_normal(K * N) * 0.3).astype(np.float32)
    st = o.quantize(W)
    w_hat = o.dequantize(st, "fp32").reshape(K, N)
    A = (rng.integers(-64, 65, (K, r)) * 2.0 ** -7).astype(np.float32)
    B = (rng.integers(-64, 65, (r, N)) * 2.0 ** -9).astype(np.float32)
    c = 0.75
    got = o.merge(st, A, B, c, K, N)
    for k in range(K):
        for n in range(N):
            s = sum(Fraction(float(A[k, t])) * Fraction(float(B[t, n])) for t in range(r))
            assert got[k, n] == exact_round_f32(Fraction(float(w_hat[k, n])) + Fraction(c) * s)
    assert np.array_equal(o.merge(st, A, B, 0.0, K, N), w_hat)
    assert np.array_equal(o.merge(st, A, np.zeros_like(B), c, K, N), w_hat)
    assert not np.array_equal(o.merge(st, A, np.zeros_like(B), c, K, N), W.reshape(K, N))


def test_sgd_page_example():
    """One step on the worked adapter with fp32 masters gives a = [0.12025,
    0.2405], b = 0.33375 (to fp32 rounding) and a lower loss."""
    g = load("p1_sgd_update.txt")
    lr = float(g["learning_rate"])
    a0 = np.array(floats(g["A"]), np.float32)
    b0 = np.array(floats(g["B"]), np.float32)
    _, a1 = o.sgd_step(a0, np.array(floats(g["dA"]), np.float32), lr, master=a0)
    _, b1 = o.sgd_step(b0, np.array(floats(g["dB"]), np.float32), lr, master=b0)
    assert np.allclose(a1, floats(g["A_updated"]), rtol=0, atol=2e-8)
    assert np.allclose(b1, floats(g["B_updated"]), rtol=0, atol=3e-8)
    e, X, W_hat, A, B, c, target = _layer_example()
    loss = lambda A_, B_: 0.5 * float((o.layer_forward(X, W_hat, A_, B_, c)[0][0, 0] - target) ** 2)
    assert loss(a1.reshape(2, 1), b1.reshape(1, 1)) < loss(A, B)


def test_sgd_exact_cases():
    """Power-of-two steps are exact; without a master the bf16 value itself is
    stepped and rounded to bf16 (ties to even)."""
    p = np.array([1.0, -0.5, 0.25, 3.0], np.float32)
    g = np.array([0.5, 0.25, -1.0, 0.0], np.float32)
    bf, new = o.sgd_step(p, g, 0.5, master=p.copy())
    assert new.tolist() == [0.75, -0.625, 0.75, 3.0] and bf.tolist() == new.tolist()
    # 1 - 2^-9: not a bf16 value; RNE to bf16 rounds to 1.0 (tie between 1 - 2^-8 and 1 -> even = 1.0)
    bf, new = o.sgd_step(np.array([1.0], np.float32), np.array([2.0 ** -8], np.float32), 0.5)
    assert new is None and bf.tolist() == [1.0]
    assert exact_round_bf16(1.0 - 2.0 ** -9) == 1.0


def _layer_example():
    g = load("p1_layer_example.txt")
    st = o.quantize(np.array(floats(g["weight"]), np.float32))
    assert st["codes_packed"].tobytes().hex() == g["payload_hex"]
    assert st["codes"].tolist() == ints(g["codes"])
    assert float(st["absmax"][0]) == float(g["scale"])
    W_hat = o.dequantize(st, "fp32").astype(np.float64).reshape(2, 1)
    X = np.array([floats(g["x"])])
    A = np.array(floats(g["A"])).reshape(2, 1)
    B = np.array(floats(g["B"])).reshape(1, 1)
    return g, X, W_hat, A, B, float(g["c"]), float(g["target"])


def test_layer_example_forward_backward():
    g, X, W_hat, A, B, c, target = _layer_example()
    Y, _ = o.layer_forward(X, W_hat, A, B, c)
    assert math.isclose(Y[0, 0], float(g["y"]), rel_tol=1e-12)
    G = Y - target
    assert math.isclose(G[0, 0], float(g["G"]), rel_tol=1e-12)
    dX, dA, dB, _ = o.layer_backward(G, X, W_hat, A, B, c)
    np.testing.assert_allclose(dX.ravel(), floats(g["dX"]), rtol=1e-12)
    np.testing.assert_allclose(dA.ravel(), floats(g["dA"]), rtol=1e-12)
    np.testing.assert_allclose(dB.ravel(), floats(g["dB"]), rtol=1e-12)
    # B = 0: dA is exactly zero while dB is not
    dX0, dA0, dB0, _ = o.layer_backward(o.layer_forward(X, W_hat, A, 0 * B, c)[0] - target,
                                        X, W_hat, A, 0 * B, c)
    assert np.all(dA0 == 0.0) and abs(dB0[0, 0]) > 0.1


def test_layer_example_finite_differences():
    g, X, W_hat, A, B, c, target = _layer_example()
    eps, rtol = float(g["fd_eps"]), float(g["fd_rel_tol"])

    def loss(params):
        x, a, b = params[:2].reshape(1, 2), params[2:4].reshape(2, 1), params[4:].reshape(1, 1)
        y = o.layer_forward(x, W_hat, a, b, c)[0][0, 0]
        return 0.5 * (y - target) ** 2

    p = np.concatenate([X.ravel(), A.ravel(), B.ravel()])
    Y, _ = o.layer_forward(X, W_hat, A, B, c)
    dX, dA, dB, _ = o.layer_backward(Y - target, X, W_hat, A, B, c)
    analytic = np.concatenate([dX.ravel(), dA.ravel(), dB.ravel()])
    for i in range(p.size):
        pp, pm = p.copy(), p.copy()
        pp[i] += eps
        pm[i] -= eps
        num = (loss(pp) - loss(pm)) / (2 * eps)
        assert math.isclose(num, analytic[i], rel_tol=rtol, abs_tol=1e-9)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_layer_gradients_finite_differences_random(seed):
    """Central differences of L = sum(Y * R) on random small shapes: dL/dY = R."""
    rng = np.random.default_rng(seed)
    M, K, N, r = 3, 5, 4, 2
    X, W, A, B, R = (rng.standard_normal(s) for s in [(M, K), (K, N), (K, r), (r, N), (M, N)])
    c = 0.7

    def L(X, A, B):
        return float(np.sum(o.layer_forward(X, W, A, B, c)[0] * R))

    dX, dA, dB, _ = o.layer_backward(R, X, W, A, B, c)
    eps = 1e-6
    for T, dT, name in ((X, dX, "X"), (A, dA, "A"), (B, dB, "B")):
        for idx in np.ndindex(T.shape):
            Tp, Tm = T.copy(), T.copy()
            Tp[idx] += eps
            Tm[idx] -= eps
            args = {"X": X, "A": A, "B": B}
            ap, am = dict(args), dict(args)
            ap[name], am[name] = Tp, Tm
            num = (L(**ap) - L(**am)) / (2 * eps)
            assert math.isclose(num, dT[idx], rel_tol=1e-6, abs_tol=1e-8), (name, idx)


# ------------------------------------------------------ nearest-code search (P1)
@pytest.mark.parametrize("seed", range(4))
def test_nf4_codes_match_exact_rational_search(seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(64 * 8) * rng.choice([1e-3, 0.02, 3.0])).astype(np.float32)
    w[::97] = 0.0
    a = o.first_level_absmax(w)
    codes = o.nf4_codes(w, a)
    for i, wi in enumerate(w):
        v = Fraction(float(wi)) / Fraction(float(a[i // 64]))
        assert codes[i] == exact_nearest(v, NF4), i


def test_nf4_codes_near_midpoints_match_exact():
    """Weights within a few ulps of every midpoint m_j * a, for many scales."""
    rng = np.random.default_rng(7)
    mids = [(NF4[j] + NF4[j + 1]) / 2 for j in range(15)]
    for a in np.concatenate([rng.uniform(1e-3, 10, 40), [1.0, 0.5, 2.0 ** -100, 3e-39]]).astype(np.float32):
        for m in mids:
            t = np.float32(float(m * Fraction(float(a))))
            w = [t]
            for _ in range(3):
                w.append(np.nextafter(w[-1], np.float32(np.inf)))
            w2 = [t]
            for _ in range(3):
                w2.append(np.nextafter(w2[-1], np.float32(-np.inf)))
            ws = np.array(w + w2[1:], np.float32)
            if np.any(np.abs(ws) > a):
                continue
            block = np.concatenate([ws, [a]]).astype(np.float32)
            aa = o.first_level_absmax(block)
            assert aa[0] == a
            codes = o.nf4_codes(block, aa)
            for i, wi in enumerate(block):
                v = Fraction(float(wi)) / Fraction(float(a))
                assert codes[i] == exact_nearest(v, NF4), (float(a), float(wi))


def test_nf4_exact_ties_go_to_smaller_index():
    """w exactly on a midpoint: the smaller code wins."""
    for j in range(15):
        m = (NF4[j] + NF4[j + 1]) / 2
        for e in range(-3, 4):
            a = Fraction(2) ** e
            t = m * a
            if Fraction(float(np.float32(float(t)))) != t:
                continue  # midpoint not representable in fp32 at this scale
            block = np.array([float(t), float(a)], np.float32)
            codes = o.nf4_codes(block, o.first_level_absmax(block))
            assert codes[0] == j, (j, e)


def test_absmax_element_gets_an_endpoint_code():
    rng = np.random.default_rng(3)
    w = rng.standard_normal(64 * 16).astype(np.float32)
    a = o.first_level_absmax(w)
    codes = o.nf4_codes(w, a)
    for b in range(16):
        blk = w[b * 64:(b + 1) * 64]
        i = int(np.argmax(np.abs(blk)))
        assert codes[b * 64 + i] == (15 if blk[i] > 0 else 0)


def test_partial_last_block_and_zero_block_inside_tensor():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal(64 * 3 + 17) * 0.02).astype(np.float32)
    w[64:128] = 0.0
    st = o.quantize(w)
    a = st["absmax"]
    assert a.size == 4 and a[1] == 1.0
    assert a[3] == np.abs(w[192:]).max()
    assert np.all(st["codes"][64:128] == 7)
    rec = o.dequantize(st, "fp32")
    assert np.all(rec[64:128] == 0.0)
    # odd length: the pad nibble is code 7
    assert (st["codes_packed"][-1] & 15) == 7


# --------------------------------------------------------- second level (P1/P2)
def test_linear_absmax_reproduces_p2_int4_example():
    g = load("p2_int4_example.txt")
    v = np.array(floats(g["input"]), np.float32)
    q, s = o.linear_absmax_codes(v, int(g["levels"]))
    assert q.tolist() == ints(g["q"])
    table = o.linear_absmax_table(int(g["levels"]))
    rec = table[q + int(g["levels"])] * s
    tol = float(g["approx_tol"])
    assert abs(float(s) / 7 - float(g["scale_approx"])) < tol
    np.testing.assert_allclose(rec, floats(g["restored_approx"]), atol=tol)


def test_linear_table_is_correctly_rounded():
    for L in (7, 127):
        t = o.linear_absmax_table(L)
        assert t.size == 2 * L + 1 and t[L] == 0 and t[0] == -1 and t[-1] == 1
        for q in range(-L, L + 1):
            assert t[q + L] == exact_round_f32(Fraction(q, L))


@pytest.mark.parametrize("seed", range(3))
def test_linear_codes_match_exact_rational_search(seed):
    rng = np.random.default_rng(100 + seed)
    vals = (rng.standard_normal(256) * 0.05).astype(np.float32)
    q, s = o.linear_absmax_codes(vals, 127)
    table = [Fraction(float(x)) for x in o.linear_absmax_table(127)]
    assert s == np.abs(vals).max()
    for i, x in enumerate(vals):
        assert q[i] + 127 == exact_nearest(Fraction(float(x)) / Fraction(float(s)), table)


def test_linear_codes_near_midpoints_and_ties():
    table = [Fraction(float(x)) for x in o.linear_absmax_table(127)]
    rng = np.random.default_rng(11)
    for s in np.concatenate([rng.uniform(1e-4, 1, 8), [1.0, 0.25]]).astype(np.float32):
        for k in range(0, 254, 7):
            t = np.float32(float((table[k] + table[k + 1]) / 2 * Fraction(float(s))))
            vals = [t, np.nextafter(t, np.float32(1)), np.nextafter(t, np.float32(-1)), s]
            vals = np.array(vals, np.float32)
            q, ss = o.linear_absmax_codes(vals, 127)
            assert ss == s
            for i, x in enumerate(vals):
                assert q[i] + 127 == exact_nearest(Fraction(float(x)) / Fraction(float(s)), table)


def test_linear_codes_zero_group():
    q, s = o.linear_absmax_codes(np.zeros(5, np.float32), 127)
    assert s == 1.0 and np.all(q == 0)


def _exact_mean_f32(a):
    return np.float32(float(sum(Fraction(float(x)) for x in a) / len(a)))


def test_tree_offset_exact_cases():
    # small dyadic values: every partial sum is exact, so the tree equals the exact mean
    rng = np.random.default_rng(2)
    for n1 in (1, 2, 3, 255, 256, 257, 1000, 4097):
        a = (rng.integers(1, 1 << 12, n1) / 1024.0).astype(np.float32)
        assert o.tree_offset(a) == _exact_mean_f32(a), n1


def test_tree_offset_error_bound():
    rng = np.random.default_rng(4)
    for n1 in (7, 300, 5000, 70000):
        a = np.abs(rng.standard_normal(n1) * 0.05).astype(np.float32) + np.float32(1e-3)
        exact = math.fsum(a.astype(np.float64)) / n1
        got = float(o.tree_offset(a))
        # fp64 tree error is ~log2(n) * 2^-53 relative; fp32 rounding dominates
        assert abs(got - exact) <= 2.0 ** -24 * exact * 1.01
        assert got == float(np.float32(exact)) or abs(got - exact) <= 2.0 ** -24 * exact


def test_double_quantize_special_cases_are_exact():
    # a single block: offset = a, centred value 0, s2 -> 1, q = 0, â = a
    for a0 in (0.5, 0.53, 1e-30, 123.25):
        a = np.array([a0], np.float32)
        q, s2, off = o.double_quantize(a)
        assert q.tolist() == [0] and s2.tolist() == [1.0]
        assert o.reconstruct_absmax(q, s2, off)[0] == np.float32(a0)
    # all blocks equal: same
    a = np.full(700, 0.0371, np.float32)
    q, s2, off = o.double_quantize(a)
    assert np.all(o.reconstruct_absmax(q, s2, off) == a)


@pytest.mark.parametrize("seed", range(3))
def test_double_quantize_error_bound(seed):
    """|â - a| <= s2/254 (half a linear step) plus the fp32 roundings."""
    rng = np.random.default_rng(seed)
    a = np.abs(rng.standard_normal(256 * 5 + 33) * 0.02).astype(np.float32) + np.float32(0.001)
    q, s2, off = o.double_quantize(a)
    ahat = o.reconstruct_absmax(q, s2, off)
    s = np.repeat(s2, 256)[: a.size].astype(np.float64)
    err = np.abs(ahat.astype(np.float64) - a.astype(np.float64))
    ulp = 2.0 ** -23 * (np.abs(a.astype(np.float64)) + s + abs(float(off)))
    assert np.all(err <= s / 254 + 2 * ulp)
    # the group absmax element is reconstructed to within roundings only
    for g in range(s2.size):
        c = (a[g * 256:(g + 1) * 256] - off).astype(np.float32)
        i = int(np.argmax(np.abs(c)))
        assert abs(int(q[g * 256 + i])) == 127


def _reconstruct_absmax_pin_holds(reconstruct, seed: int = 0) -> bool:
    """The exact-rational pin of the scale reconstruction for a given
    function: â = fl32(fl32(Q[q] s2) + offset), each rounding taken on the
    exact rational value ([P1] "Double Quantization 压缩的是 Scale": decode
    the second level, then add the offset back; reading R4).  The inputs mix
    offsets of the size of the decoded values, so that one rounding instead
    of two, or an unrounded table value, changes many results."""
    rng = np.random.default_rng(100 + seed)
    n1 = 256 * 6 + 17
    q = rng.integers(-127, 128, n1).astype(np.int8)
    s2 = (np.abs(rng.standard_normal(7)) * 0.05 + 1e-3).astype(np.float32)
    table = o.linear_absmax_table(127)
    for off in (np.float32(0.031), np.float32(-0.0173), np.float32(rng.uniform(0.001, 0.2))):
        got = reconstruct(q, s2, off)
        for i in range(n1):
            prod = exact_round_f32(Fraction(float(table[int(q[i]) + 127])) * Fraction(float(s2[i // 256])))
            if got[i] != exact_round_f32(Fraction(float(prod)) + Fraction(float(off))):
                return False
    return True


@pytest.mark.parametrize("seed", range(2))
def test_reconstruct_absmax_two_exact_roundings(seed):
    assert _reconstruct_absmax_pin_holds(o.reconstruct_absmax, seed)


def test_reconstruct_absmax_pin_catches_one_rounding():
    """Plausible mistakes in the scale reconstruction fail the exact pin:
    the whole expression in float64 rounded once (a fused multiply-add),
    and the code value q/127 used unrounded."""
    table = o.linear_absmax_table(127)

    def one_rounding(q, s2, off):
        qv = table[np.asarray(q, np.int64) + 127].astype(np.float64)
        s = np.repeat(np.asarray(s2, np.float64), 256)[: qv.size]
        return (qv * s + np.float64(off)).astype(np.float32)

    def unrounded_code(q, s2, off):
        qv = np.asarray(q, np.int64) / 127.0
        s = np.repeat(np.asarray(s2, np.float64), 256)[: qv.size]
        return ((qv * s).astype(np.float32) + np.float32(off)).astype(np.float32)

    for bad in (one_rounding, unrounded_code):
        assert not _reconstruct_absmax_pin_holds(bad), bad.__name__


# ------------------------------------------------------------------ bf16 (R5)
def test_bf16_round_matches_exact_rne():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(2000) * np.exp(rng.uniform(-20, 20, 2000))).astype(np.float32)
    # include exact ties (lower 16 bits = 0x8000) with both parities of bit 16
    m = rng.integers(0, 64, 100).astype(np.uint32)
    par = (np.arange(100) % 2).astype(np.uint32)
    ties = (np.uint32(0x3F000000) | (m << np.uint32(17)) | (par << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)
    ties2 = -ties
    x = np.concatenate([x, ties, ties2]).astype(np.float32)
    got = o.bf16_round(x)
    for xi, gi in zip(x, got):
        assert float(gi) == exact_round_bf16(float(xi))


def test_bf16_of_worked_block_values():
    # derived: RNE of the fp32 reconstructions of codes 9 and 3 at scale 1
    got = o.bf16_round(np.array([0.16093020141124725, -0.39491748809814453], np.float32))
    assert got.tolist() == [0.1611328125, -0.39453125]


# -------------------------------------------------------------- storage bill
def test_storage_bits_closed_forms():
    g = load("p1_storage.txt")
    P = 16384 * 4096
    assert o.storage_bits(P, double_quant=False) / P == float(g["no_dq_total_bits"])
    assert (o.storage_bits(P, False) - 4 * P) / P == float(g["scale_only_bits"])
    dq = (o.storage_bits(P) - 32) / P
    assert dq == float(g["dq_asymptote_bits"])
    assert float(g["no_dq_total_bits"]) - dq == float(g["dq_saving_bits"])
    assert round(dq - 4, 3) == float(g["dq_overhead_rounded"])
    # small tensors: exact bill with ceilings
    assert o.storage_bits(1) == 8 + 8 + 32 + 32
    assert o.storage_bits(65) == 8 * 33 + 8 * 2 + 32 + 32
    assert o.counts(64 * 256 + 1) == (257, 2)


# ------------------------------------------------ the pins catch planted bugs
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle and check a pin fails for each."""
    w = np.array([0.0, 0.2, -0.4, 1.0], np.float32)

    def worked_block_ok():
        st = o.quantize(w)
        return (st["codes"].tolist() == [7, 9, 3, 15]
                and st["codes_packed"].tobytes().hex() == "793f")

    assert worked_block_ok()
    # 1. nibble order swapped
    orig_pack = o.pack_nibbles
    monkeypatch.setattr(o, "pack_nibbles",
                        lambda c: ((lambda p, L: (((p & 15) << 4 | p >> 4).astype(np.uint8), L))(*orig_pack(c))))
    assert not worked_block_ok()
    monkeypatch.setattr(o, "pack_nibbles", orig_pack)
    # 2. ties to the larger index
    orig_nearest = o._nearest
    monkeypatch.setattr(o, "_nearest", lambda v, t: (t.size - 1) - np.argmin(np.abs(v[:, None] - t[None, ::-1]), axis=1))
    block = np.array([float((NF4[7] + NF4[8]) / 2), 1.0], np.float32)
    assert o.nf4_codes(block, o.first_level_absmax(block))[0] != 7
    monkeypatch.setattr(o, "_nearest", orig_nearest)
    # 3. layer mistakes: dB without c, a transposed operand in dX, a dropped term
    def bwd_no_c(G, X, W, A, B, c):
        dX, dA, dB, dZ = o.layer_backward(G, X, W, A, B, c)
        return dX, dA, dB / c, dZ

    def bwd_dropped_term(G, X, W, A, B, c):
        dX, dA, dB, dZ = o.layer_backward(G, X, W, A, B, c)
        return dX - dZ @ np.asarray(A).T, dA, dB, dZ

    def bwd_transposed(G, X, W, A, B, c):
        dX, dA, dB, dZ = o.layer_backward(G, X, W, A, B, c)
        return dX, np.asarray(X).T @ np.flipud(dZ), dB, dZ

    assert _fd_agrees(o.layer_backward)
    for bad in (bwd_no_c, bwd_dropped_term, bwd_transposed):
        assert not _fd_agrees(bad), bad.__name__
    # 4. merge mistakes: the raw W instead of Ŵ, c dropped, B's columns reversed
    orig_merge = o.merge

    def merge_raw_w(state, A, B, c, K, N):
        w = state["_W_for_planted_test"].astype(np.float64).reshape(K, N)
        inc = np.asarray(A, np.float64) @ np.asarray(B, np.float64)
        return (w + c * inc).astype(np.float32)

    def merge_no_c(state, A, B, c, K, N):
        return orig_merge(state, A, B, 1.0, K, N)

    def merge_flipped(state, A, B, c, K, N):
        return orig_merge(state, A, np.asarray(B)[:, ::-1], c, K, N)

    assert _merge_pins_hold(orig_merge)
    for bad in (merge_raw_w, merge_no_c, merge_flipped):
        assert not _merge_pins_hold(bad), bad.__name__
    # 5. the scale reconstruction rounded once (float64, then one fl32)
    def reconstruct_once(q, s2, off):
        qv = o.linear_absmax_table(127)[np.asarray(q, np.int64) + 127].astype(np.float64)
        s = np.repeat(np.asarray(s2, np.float64), 256)[: qv.size]
        return (qv * s + np.float64(off)).astype(np.float32)

    monkeypatch.setattr(o, "reconstruct_absmax", reconstruct_once)
    assert not _reconstruct_absmax_pin_holds(o.reconstruct_absmax)


def _merge_pins_hold(merge) -> bool:
    """The exact-rational merge pin (c = 0.75, integer-scaled values) and
    the c = 0 case, for a given merge function."""
    rng = np.random.default_rng(11)
    K, N, r = 3, 64, 5
    W = (rng.standard_normal(K * N) * 0.3).astype(np.float32)
    st = dict(o.quantize(W))
    st["_W_for_planted_test"] = W
    w_hat = o.dequantize(st, "fp32").reshape(K, N)
    A = (rng.integers(-64, 65, (K, r)) * 2.0 ** -7).astype(np.float32)
    B = (rng.integers(-64, 65, (r, N)) * 2.0 ** -9).astype(np.float32)
    got = merge(st, A, B, 0.75, K, N)
    for k in range(K):
        for n in range(N):
            s = sum(Fraction(float(A[k, t])) * Fraction(float(B[t, n])) for t in range(r))
            if got[k, n] != exact_round_f32(Fraction(float(w_hat[k, n])) + Fraction(0.75) * s):
                return False
    return bool(np.array_equal(merge(st, A, B, 0.0, K, N), w_hat))


def _fd_agrees(backward) -> bool:
    rng = np.random.default_rng(42)
    M, K, N, r = 3, 4, 5, 2
    X, W, A, B, R = (rng.standard_normal(s) for s in [(M, K), (K, N), (K, r), (r, N), (M, N)])
    c = 0.7

    def L(X, A, B):
        return float(np.sum(o.layer_forward(X, W, A, B, c)[0] * R))

    grads = dict(zip("XAB", backward(R, X, W, A, B, c)[:3]))
    args = {"X": X, "A": A, "B": B}
    for name, T in args.items():
        for idx in np.ndindex(T.shape):
            ap, am = dict(args), dict(args)
            ap[name] = T.copy(); ap[name][idx] += 1e-6
            am[name] = T.copy(); am[name][idx] -= 1e-6
            num = (L(**ap) - L(**am)) / 2e-6
            if not math.isclose(num, grads[name][idx], rel_tol=1e-6, abs_tol=1e-8):
                return False
    return True
