"""The no-allocation forward (qlora_linear_fwd_noalloc): called through the C
ABI on two calls in a row, the second with a smaller input, it returns the
same bits as qlora_linear_fwd with a caller workspace; and shapes whose
forward workspace exceeds the library's scratch are rejected."""
import ctypes

import numpy as np
import pytest

import bit_nf4_quantized_10_amd as qn
import synth_inputs as si
from tests.gpu_util import dev_bf16, host, say

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, r, seed):
    import torch
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    state, status = qn.nf4_quantize(torch.from_numpy(W).cuda().reshape(-1))
    assert qn.nf4_status_read(status) == 0
    X = dev_bf16(si.bf16_normal((M, K), 1.0, seed + 1)[0])
    A = dev_bf16(si.bf16_normal((K, r), 1.0 / r, seed + 2)[0])
    B = dev_bf16(si.bf16_normal((r, N), 0.01, seed + 3)[0])
    return state, X, A, B


def _both(M, K, N, r, c, seed):
    import torch
    state, X, A, B = _inputs(M, K, N, r, seed)
    Y0, Z0 = qn.qlora_linear_fwd(X, state, A, B, c, K, N)
    Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    Z1 = torch.full((M, r), float("nan"), dtype=torch.bfloat16, device="cuda")
    qn.qlora_linear_fwd_noalloc(X, state, A, B, c, K, N, Y1, Z1)
    # Z = NULL: Z computed in the scratch, Y the same
    Y2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    qn.qlora_linear_fwd_noalloc(X, state, A, B, c, K, N, Y2, None)
    torch.cuda.synchronize()
    return [host(t).tobytes() for t in (Y0, Z0, Y0)], [host(t).tobytes() for t in (Y1, Z1, Y2)]


@pytest.mark.parametrize("first,second", [
    ((16, 8192, 22016, 64, 0.25), (8, 1024, 2048, 16, 0.5)),     # dequant-GEMV, the 65B decode shape first
    ((130, 2048, 1536, 32, 0.5), (17, 512, 640, 8, 2.0)),        # fused-decode path, split reductions
])
def test_noalloc_matches_workspace_forward(first, second):
    for shape, seed in ((first, 11), (second, 12)):
        M, K, N, r, c = shape
        assert qn.qlora_workspace_bytes(M, K, N, r)[0] <= qn.NF4_NOALLOC_SCRATCH_BYTES
        say(f"no-alloc forward M={M} K={K} N={N} r={r}")
        want, got = _both(M, K, N, r, c, seed)
        assert got == want


def test_noalloc_rejects_shapes_beyond_its_scratch():
    import torch
    M, K, N, r = 4096, 4096, 4096, 64      # the M >= 192 forward holds the dequantized weight
    assert qn.qlora_workspace_bytes(M, K, N, r)[0] > qn.NF4_NOALLOC_SCRATCH_BYTES
    state, X, A, B = _inputs(M, K, N, r, 3)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    st = state.c_struct()
    rc = qn.lib().qlora_linear_fwd_noalloc(M, K, N, r, X.data_ptr(), ctypes.byref(st), A.data_ptr(), B.data_ptr(),
                                           ctypes.c_float(0.25), Y.data_ptr(), None, None)
    assert rc == qn.NF4_EINVAL
