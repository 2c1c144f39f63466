"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, the size queries match the pages' closed forms, and argument
errors are rejected before anything is launched.  No GPU work is issued."""
import ctypes
import os
import re

import pytest

import bit_nf4_quantized_10_amd as qn
from oracle import nf4_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert "nf4_quantize" in declared and "qlora_linear_bwd" in declared
    L = qn.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(qn.C_FUNCTIONS) == declared


@pytest.mark.parametrize("P", [1, 2, 3, 63, 64, 65, 4096, 16384, 16385, 4096 * 4096, 8192 * 22016])
def test_nf4_sizes_match_storage_bill(P):
    s = qn.nf4_sizes(P)
    n1, n2 = o.counts(P)
    assert (s["n1"], s["n2"], s["code_bytes"]) == (n1, n2, (P + 1) // 2)
    bits = 8 * s["code_bytes"] + 8 * s["n1"] + 32 * s["n2"] + 32
    assert bits == o.storage_bits(P)
    assert s["quant_workspace_bytes"] >= 4 * n1 + 8 * n2


def test_nf4_sizes_rejects_empty():
    with pytest.raises(qn.NF4Error) as e:
        qn.nf4_sizes(0)
    assert e.value.code == qn.NF4_EINVAL


@pytest.mark.parametrize("shape", [(0, 64, 64, 8), (4, 64, 63, 8), (4, 12, 64, 8), (4, 64, 64, 4),
                                   (4, 64, 64, 264), (4, 0, 64, 8),
                                   (1 << 20, 1 << 9, 64, 8),       # X of 2^29 elements (1 GiB)
                                   (4, 1 << 15, 1 << 14, 8),       # weight of 2^29 elements
                                   (1 << 16, 64, 1 << 13, 8),      # Y of 2^29 elements
                                   (1, 8, 1 << 21, 256),           # B (r x N) of 2^29 elements
                                   (1, 1 << 21, 64, 256)])         # A (K x r) of 2^29 elements
def test_layer_shapes_rejected(shape):
    with pytest.raises(qn.NF4Error):
        qn.qlora_workspace_bytes(*shape)


def test_layer_workspace_sizes_are_positive():
    for shape in [(16, 256, 256, 8), (4096, 4096, 4096, 64), (1, 8192, 22016, 64), (2048, 22016, 8192, 64),
                  ((1 << 20) - 8, 256, 64, 8)]:
        f, b = qn.qlora_workspace_bytes(*shape)
        assert f >= 0 and b > 0 and f % 256 == 0 and b % 256 == 0


def test_mid_size_workspace_holds_split_partials():
    # too few 256 x 256 output tiles to occupy the device: the GEMMs split
    # their reduction and the workspace holds at least two fp32 partial
    # copies of the output (Y for the forward, dX for the backward)
    M, K, N, r = 256, 4096, 4096, 64
    f, b = qn.qlora_workspace_bytes(M, K, N, r)
    assert f >= 2 * M * N * 4 and b >= 2 * M * K * 4
    # a full device of tiles: no partials (the forward needs far less)
    f_big, _ = qn.qlora_workspace_bytes(4096, K, N, r)
    assert f_big < 4096 * N * 4


def test_entry_points_reject_bad_arguments_before_launch():
    L = qn.lib()
    st = qn._State(64, 0x1000, 0x2000, 0x3000, 0x4000)
    # NULL weights / state / workspace / status
    assert L.nf4_quantize(None, ctypes.byref(st), 0x10000, 1 << 20, 0x5000, None) == qn.NF4_EINVAL
    assert L.nf4_quantize(0x100, None, 0x10000, 1 << 20, 0x5000, None) == qn.NF4_EINVAL
    # misaligned weights, too small a workspace
    assert L.nf4_quantize(0x104, ctypes.byref(st), 0x10000, 1 << 20, 0x5000, None) == qn.NF4_EINVAL
    assert L.nf4_quantize(0x100, ctypes.byref(st), 0x10000, 8, 0x5000, None) == qn.NF4_EINVAL
    # bad output dtype for the decoder
    assert L.nf4_dequantize(ctypes.byref(st), 0x100, 7, None, None) == qn.NF4_EINVAL
    # state buffers moved as words: misaligned codes / second-level codes / scales
    for bad_state in (qn._State(64, 0x1004, 0x2000, 0x3000, 0x4000), qn._State(64, 0x1000, 0x2001, 0x3000, 0x4000),
                      qn._State(64, 0x1000, 0x2000, 0x3002, 0x4000),
                      qn._State(64, 0x1000, None, None, None, 0x5002),     # single level, misaligned scales
                      qn._State(64, 0x1000, None, 0x3000, 0x4000, None)):  # double quantized without codes q
        assert L.nf4_quantize(0x100, ctypes.byref(bad_state), 0x10000, 1 << 20, 0x5000, None) == qn.NF4_EINVAL
        assert L.nf4_dequantize(ctypes.byref(bad_state), 0x100, qn.NF4_OUT_F32, None, None) == qn.NF4_EINVAL
    # layer: numel mismatch, N % 64, NULL output
    st2 = qn._State(64 * 64, 0x1000, 0x2000, 0x3000, 0x4000)
    args = (0x100, ctypes.byref(st2), 0x200, 0x300, ctypes.c_float(1.0), 0x400, 0x500, 0x10000, 1 << 30, None)
    assert L.qlora_linear_fwd(4, 64, 32, 8, *args) == qn.NF4_EINVAL
    assert L.qlora_linear_fwd(4, 32, 64, 8, *args) == qn.NF4_EINVAL
    bad = (0x100, ctypes.byref(st2), 0x200, 0x300, ctypes.c_float(1.0), None, 0x500, 0x10000, 1 << 30, None)
    assert L.qlora_linear_fwd(4, 64, 64, 8, *bad) == qn.NF4_EINVAL
    small_ws = (0x100, ctypes.byref(st2), 0x200, 0x300, ctypes.c_float(1.0), 0x400, 0x500, 0x10000, 0, None)
    f, _ = qn.qlora_workspace_bytes(4, 64, 64, 8)
    if f > 0:
        assert L.qlora_linear_fwd(4, 64, 64, 8, *small_ws) == qn.NF4_EINVAL
    assert L.qlora_linear_bwd(4, 64, 64, 8, 0x100, 0x100, 0x100, ctypes.byref(st2), 0x200, 0x300,
                              ctypes.c_float(1.0), None, None, 0x600, 0x10000, 1 << 30, None) == qn.NF4_EINVAL
    # Z may be NULL (computed / recomputed in the workspace), but a given Z must be aligned
    mis_z = (0x100, ctypes.byref(st2), 0x200, 0x300, ctypes.c_float(1.0), 0x400, 0x502, 0x10000, 1 << 30, None)
    assert L.qlora_linear_fwd(4, 64, 64, 8, *mis_z) == qn.NF4_EINVAL
    assert L.qlora_linear_bwd(4, 64, 64, 8, 0x100, 0x100, 0x502, ctypes.byref(st2), 0x200, 0x300,
                              ctypes.c_float(1.0), None, 0x600, 0x700, 0x10000, 1 << 30, None) == qn.NF4_EINVAL


def test_timer_ids_validated():
    L = qn.lib()
    assert L.qlora_timer_enable(99, 1) == qn.NF4_EINVAL
    assert L.qlora_timer_enable(-1, 1) == qn.NF4_EINVAL
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert L.qlora_timer_read(3, ctypes.byref(ms), ctypes.byref(n)) == qn.NF4_OK and n.value == 0


def test_error_strings():
    L = qn.lib()
    for code in (0, 1, 2, 4, 8, 6):
        assert L.nf4_error_string(code)


def test_adapter_entry_points_reject_bad_arguments():
    L = qn.lib()
    st = qn._State(64 * 64, 0x1000, 0x2000, 0x3000, 0x4000)
    ok = (64, 64, 8, ctypes.byref(st), 0x100, 0x200, qn.NF4_AB_BF16, ctypes.c_float(1.0), 0x300, None)
    bad_cases = [
        (64, 32, 8) + ok[3:],                                   # numel != K*N
        (64, 64, 0) + ok[3:],                                   # r = 0
        ok[:6] + (7,) + ok[7:],                                 # unknown A/B dtype
        ok[:4] + (None,) + ok[5:],                              # NULL A
        ok[:8] + (0x304,) + ok[9:],                             # misaligned output
        ok[:4] + (0x102,) + (ok[5], qn.NF4_AB_F32) + ok[7:],    # fp32 A not 4-byte aligned
    ]
    for args in bad_cases:
        assert L.qlora_merge(*args) == qn.NF4_EINVAL, args
    sgd_ok = (64, 64, 8, 0x100, 0x200, 0x300, 0x400, ctypes.c_float(0.1), None, None, None)
    for args in [(0, 64, 8) + sgd_ok[3:], sgd_ok[:3] + (None,) + sgd_ok[4:],
                 sgd_ok[:8] + (0x500, None, None),                # one master without the other
                 sgd_ok[:5] + (0x302,) + sgd_ok[6:]]:             # misaligned fp32 gradient
        assert L.qlora_sgd_step(*args) == qn.NF4_EINVAL, args


def test_grouped_entry_points_reject_bad_arguments():
    L = qn.lib()
    i64 = ctypes.c_int64

    def ws(M, K, Ns, r):
        f, b = i64(), i64()
        return L.qlora_grouped_workspace_bytes(M, K, len(Ns), (i64 * max(len(Ns), 1))(*Ns), r,
                                               ctypes.byref(f), ctypes.byref(b))

    assert ws(64, 256, [256, 512], 8) == qn.NF4_OK
    for M, K, Ns, r in [(64, 256, [256, 320], 8),        # a member not a multiple of 256 columns
                        (64, 256, [], 8),                # no member
                        (64, 256, [256] * 9, 8),         # more than 8 members
                        (64, 256, [256, 256], 160),      # g r above 256
                        (64, 12, [256], 8)]:             # K % 8
        assert ws(M, K, Ns, r) == qn.NF4_EINVAL, (M, K, Ns, r)
    states = (qn._State * 2)(qn._State(256 * 256, 0x1000, 0x2000, 0x3000, 0x4000),
                             qn._State(256 * 128, 0x1000, 0x2000, 0x3000, 0x4000))   # numel != K * N[1]
    Ns = (i64 * 2)(256, 256)
    assert L.qlora_grouped_fwd(8, 256, 2, Ns, 8, 0x100, states, 0x200, 0x300, ctypes.c_float(1.0), 0x400, 0x500,
                               0x10000, 1 << 30, None) == qn.NF4_EINVAL


def test_grouped_dt_entry_points_reject_unknown_compute_type():
    """qlora_grouped_fwd_dt / _bwd_dt take NF4_COMPUTE_BF16 or NF4_COMPUTE_F16
    only; anything else is rejected before any launch."""
    L = qn.lib()
    i64 = ctypes.c_int64
    Ns = (i64 * 2)(256, 256)
    states = (qn._State * 2)(*[qn._State(256 * 256, 0x1000, 0x2000, 0x3000, 0x4000) for _ in range(2)])
    for dt in (-1, 2, 7):
        assert L.qlora_grouped_fwd_dt(dt, 8, 256, 2, Ns, 8, 0x100, states, 0x200, 0x300, ctypes.c_float(1.0),
                                      0x400, 0x500, 0x10000, 1 << 30, None) == qn.NF4_EINVAL
        assert L.qlora_grouped_bwd_dt(dt, 8, 256, 2, Ns, 8, 0x100, 0x100, 0x500, states, 0x200, 0x300,
                                      ctypes.c_float(1.0), None, 0x600, 0x700, 0x10000, 1 << 30,
                                      None) == qn.NF4_EINVAL


@pytest.mark.parametrize("g,r", [(2, 4), (4, 2), (8, 1), (2, 12), (3, 20)])
def test_grouped_member_rank_must_be_a_multiple_of_8(g, r):
    """Per-member ranks that are not multiples of 8 are rejected by all three
    grouped calls even when g r is: the kernels move the concatenated Z, A,
    (c B)ᵀ and dB partials in 8-element chunks, which would then mix two
    members."""
    L = qn.lib()
    i64 = ctypes.c_int64
    K = 256
    Ns = (i64 * g)(*([256] * g))
    f, b = i64(), i64()
    assert L.qlora_grouped_workspace_bytes(64, K, g, Ns, 8, ctypes.byref(f), ctypes.byref(b)) == qn.NF4_OK
    assert L.qlora_grouped_workspace_bytes(64, K, g, Ns, r, ctypes.byref(f), ctypes.byref(b)) == qn.NF4_EINVAL
    states = (qn._State * g)(*[qn._State(K * 256, 0x1000, 0x2000, 0x3000, 0x4000) for _ in range(g)])
    assert L.qlora_grouped_fwd(64, K, g, Ns, r, 0x100, states, 0x200, 0x300, ctypes.c_float(1.0), 0x400, 0x500,
                               0x10000, 1 << 30, None) == qn.NF4_EINVAL
    assert L.qlora_grouped_bwd(64, K, g, Ns, r, 0x100, 0x100, 0x500, states, 0x200, 0x300, ctypes.c_float(1.0),
                               None, 0x600, 0x700, 0x10000, 1 << 30, None) == qn.NF4_EINVAL


def test_read_probe_library_exports_its_header_and_validates():
    """libqlora_probe.so (the read-ceiling helper of the benchmark) exports
    what include/qlora_read_probe.h declares and rejects bad arguments
    before launching anything."""
    from bit_nf4_quantized_10_amd import probe
    text = open(os.path.join(ROOT, "include", "qlora_read_probe.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    declared = sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))
    assert declared == sorted(probe.C_FUNCTIONS)
    L = probe.lib()
    for args in [(None, 1024, 256, 0x100, None), (0x100, 8, 256, 0x100, None), (0x100, 1000, 256, 0x100, None),
                 (0x100, 1024, 0, 0x100, None), (0x108, 1024, 256, 0x100, None), (0x100, 1024, 256, None, None)]:
        assert L.qlora_read_probe(*args) == 1, args
