"""Python binding of the MI355X QLoRA NF4 library (libqlora_nf4.so).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/qlora_nf4.h.  PyTorch provides device
memory and the current stream.  There is no CPU fallback: if the library is
not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqlora_nf4.so")

NF4_OK, NF4_EINVAL, NF4_ENONFINITE, NF4_EPADDING, NF4_EHIP = 0, 1, 2, 4, 8
NF4_OUT_F32, NF4_OUT_BF16, NF4_OUT_F16 = 0, 1, 2
NF4_COMPUTE_BF16, NF4_COMPUTE_F16 = 0, 1
KERNEL_IDS = {
    "quant_pass1": 0, "quant_mean": 1, "quant_pass2": 2, "dequant": 3, "lora_down": 4,
    "fwd_gemm": 5, "fwd_gemv": 6, "bwd_dz": 7, "bwd_dx": 8, "bwd_colsum": 9, "dequant_bf16": 10,
    "reduce": 11, "merge": 12, "sgd": 13,
}
C_FUNCTIONS = [
    "nf4_sizes", "nf4_quantize", "nf4_dequantize", "qlora_workspace_bytes",
    "qlora_linear_fwd", "qlora_linear_bwd", "nf4_status_read", "qlora_timer_enable",
    "qlora_timer_read", "qlora_merge", "qlora_sgd_step", "qlora_grouped_workspace_bytes",
    "qlora_grouped_fwd", "qlora_grouped_bwd", "qlora_linear_fwd_dt", "qlora_linear_bwd_dt", "qlora_sgd_step_dt",
    "qlora_linear_fwd_noalloc", "qlora_grouped_fwd_dt", "qlora_grouped_bwd_dt", "nf4_error_string",
]
NF4_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024


class NF4Error(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: error {code}")
        self.code = code


class _State(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("codes", ctypes.c_void_p), ("qabsmax", ctypes.c_void_p),
                ("absmax2", ctypes.c_void_p), ("offset", ctypes.c_void_p), ("absmax", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_nf4_quantized_10_amd.build_lib`")
        # PyTorch brings its own HIP and HSA runtimes.  Loaded first, they
        # satisfy this library's libamdhip64 dependency, so the process holds
        # one HSA runtime; loaded the other way round, the process ends up
        # with two, and the second cannot reach the GPU.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, i32p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        sp = ctypes.POINTER(_State)
        L.nf4_sizes.argtypes = [i64] + [ctypes.POINTER(i64)] * 4
        L.nf4_quantize.argtypes = [vp, sp, vp, i64, i32p, vp]
        L.nf4_dequantize.argtypes = [sp, vp, ctypes.c_int, i32p, vp]
        L.qlora_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.qlora_linear_fwd.argtypes = [i64, i64, i64, i64, vp, sp, vp, vp, ctypes.c_float, vp, vp, vp, i64, vp]
        L.qlora_linear_bwd.argtypes = [i64, i64, i64, i64, vp, vp, vp, sp, vp, vp, ctypes.c_float,
                                       vp, vp, vp, vp, i64, vp]
        L.nf4_status_read.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), vp]
        L.qlora_timer_enable.argtypes = [ctypes.c_int, ctypes.c_int]
        L.qlora_timer_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
        L.qlora_merge.argtypes = [i64, i64, i64, sp, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp]
        L.qlora_sgd_step.argtypes = [i64, i64, i64, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]
        i64p = ctypes.POINTER(i64)
        L.qlora_grouped_workspace_bytes.argtypes = [i64, i64, ctypes.c_int, i64p, i64, i64p, i64p]
        L.qlora_grouped_fwd.argtypes = [i64, i64, ctypes.c_int, i64p, i64, vp, sp, vp, vp, ctypes.c_float,
                                        vp, vp, vp, i64, vp]
        L.qlora_grouped_bwd.argtypes = [i64, i64, ctypes.c_int, i64p, i64, vp, vp, vp, sp, vp, vp, ctypes.c_float,
                                        vp, vp, vp, vp, i64, vp]
        L.qlora_linear_fwd_dt.argtypes = [ctypes.c_int] + L.qlora_linear_fwd.argtypes
        L.qlora_linear_bwd_dt.argtypes = [ctypes.c_int] + L.qlora_linear_bwd.argtypes
        L.qlora_sgd_step_dt.argtypes = [ctypes.c_int] + L.qlora_sgd_step.argtypes
        L.qlora_linear_fwd_noalloc.argtypes = [i64, i64, i64, i64, vp, sp, vp, vp, ctypes.c_float, vp, vp, vp]
        L.qlora_grouped_fwd_dt.argtypes = [ctypes.c_int] + L.qlora_grouped_fwd.argtypes
        L.qlora_grouped_bwd_dt.argtypes = [ctypes.c_int] + L.qlora_grouped_bwd.argtypes
        L.nf4_error_string.argtypes = [ctypes.c_int]
        L.nf4_error_string.restype = ctypes.c_char_p
        for name in C_FUNCTIONS[:-1]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != NF4_OK:
        raise NF4Error(rc, f"{what} ({lib().nf4_error_string(rc).decode()})")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _require_cuda(t, name: str, dtype=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


@dataclass
class NF4State:
    """Frozen NF4 state of one weight tensor (device tensors).  Double
    quantized: qabsmax / absmax2 / offset set, absmax None.  Single level
    (double quantization off): absmax set, the other three None."""
    numel: int
    codes: "torch.Tensor"             # uint8[ceil(P/2)]
    qabsmax: "torch.Tensor | None"    # int8[n1]
    absmax2: "torch.Tensor | None"    # float32[n2]
    offset: "torch.Tensor | None"     # float32[1]
    absmax: "torch.Tensor | None" = None   # float32[n1]

    @property
    def double_quant(self) -> bool:
        return self.absmax is None

    def c_struct(self) -> _State:
        return _State(self.numel, self.codes.data_ptr(), _ptr(self.qabsmax), _ptr(self.absmax2),
                      _ptr(self.offset), _ptr(self.absmax))


def nf4_sizes(numel: int) -> dict:
    out = [ctypes.c_int64() for _ in range(4)]
    _check(lib().nf4_sizes(numel, *[ctypes.byref(o) for o in out]), "nf4_sizes")
    return dict(zip(("code_bytes", "n1", "n2", "quant_workspace_bytes"), (o.value for o in out)))


def empty_state(numel: int, device="cuda", double_quant: bool = True) -> NF4State:
    import torch
    s = nf4_sizes(numel)
    codes = torch.empty(s["code_bytes"], dtype=torch.uint8, device=device)
    if not double_quant:
        return NF4State(numel, codes, None, None, None, torch.empty(s["n1"], dtype=torch.float32, device=device))
    return NF4State(numel, codes,
                    torch.empty(s["n1"], dtype=torch.int8, device=device),
                    torch.empty(s["n2"], dtype=torch.float32, device=device),
                    torch.empty(1, dtype=torch.float32, device=device))


def nf4_quantize(W, state: NF4State | None = None, workspace=None, status=None, stream=None,
                 double_quant: bool = True):
    """Encode fp32 weights (any shape, flattened row-major) into an NF4State
    (single level when double_quant is False or the given state has absmax).
    Returns (state, status) where status is the device int32 status word."""
    import torch
    _require_cuda(W, "W", torch.float32)
    P = W.numel()
    if state is None:
        state = empty_state(P, W.device, double_quant)
    sizes = nf4_sizes(P)
    if workspace is None:
        workspace = torch.empty(sizes["quant_workspace_bytes"], dtype=torch.uint8, device=W.device)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=W.device)
    st = state.c_struct()
    _check(lib().nf4_quantize(W.data_ptr(), ctypes.byref(st), workspace.data_ptr(), workspace.numel(),
                              status.data_ptr(), _stream(stream)), "nf4_quantize")
    return state, status


def nf4_dequantize(state: NF4State, out_dtype: str = "bf16", out=None, status=None, stream=None):
    """ŵ as fp32 ("fp32"), bf16 ("bf16") or fp16 ("f16")."""
    import torch
    dt, code = {"bf16": (torch.bfloat16, NF4_OUT_BF16), "f16": (torch.float16, NF4_OUT_F16),
                "fp32": (torch.float32, NF4_OUT_F32)}[out_dtype]
    if out is None:
        out = torch.empty(state.numel, dtype=dt, device=state.codes.device)
    st = state.c_struct()
    _check(lib().nf4_dequantize(ctypes.byref(st), out.data_ptr(), code, _ptr(status), _stream(stream)),
           "nf4_dequantize")
    return out


def _group_args(states, Ns):
    g = len(Ns)
    if len(states) != g or not 1 <= g <= 8:
        raise ValueError("one state per member, 1 to 8 members")
    return g, (ctypes.c_int64 * g)(*Ns), (_State * g)(*[s.c_struct() for s in states])


def qlora_grouped_workspace_bytes(M: int, K: int, Ns, r: int) -> tuple[int, int]:
    f, b = ctypes.c_int64(), ctypes.c_int64()
    arr = (ctypes.c_int64 * len(Ns))(*Ns)
    _check(lib().qlora_grouped_workspace_bytes(M, K, len(Ns), arr, r, ctypes.byref(f), ctypes.byref(b)),
           "qlora_grouped_workspace_bytes")
    return f.value, b.value


def qlora_grouped_fwd(X, states, A, B, c: float, K: int, Ns, Y=None, Z=None, workspace=None, stream=None):
    """Members sharing X, side by side: A = [A_i] (K x g r), B = [B_i] (r x sum N),
    returns (Y = [Y_i] (M x sum N), Z = [Z_i] (M x g r)).  The compute type is
    X's dtype (bf16 or fp16); A, B, Y and Z share it."""
    import torch
    g, Narr, Sarr = _group_args(states, Ns)
    M = X.shape[0]
    r = A.shape[1] // g
    Ntot = sum(Ns)
    dt = _compute_dtype(X)
    for t, n in ((X, "X"), (A, "A"), (B, "B")):
        _require_cuda(t, n, dt)
    if Y is None:
        Y = torch.empty(M, Ntot, dtype=dt, device=X.device)
    if Z is None:
        Z = torch.empty(M, g * r, dtype=dt, device=X.device)
    _require_cuda(Y, "Y", dt)
    _require_cuda(Z, "Z", dt)
    if workspace is None:
        workspace = torch.empty(max(qlora_grouped_workspace_bytes(M, K, Ns, r)[0], 256), dtype=torch.uint8,
                                device=X.device)
    _check(lib().qlora_grouped_fwd_dt(_COMPUTE[dt], M, K, g, Narr, r, X.data_ptr(), Sarr, A.data_ptr(),
                                      B.data_ptr(), ctypes.c_float(c), Y.data_ptr(), Z.data_ptr(),
                                      workspace.data_ptr(), workspace.numel(), _stream(stream)),
           "qlora_grouped_fwd_dt")
    return Y, Z


def qlora_grouped_bwd(G, X, Z, states, A, B, c: float, K: int, Ns, need_dx: bool = True, dX=None, dA=None,
                      dB=None, workspace=None, stream=None):
    """Returns (dX or None, dA = [dA_i] (K x g r fp32), dB = [dB_i] (r x sum N fp32)).
    The compute type is X's dtype (bf16 or fp16); G, Z, A, B and dX share it."""
    import torch
    g, Narr, Sarr = _group_args(states, Ns)
    M = X.shape[0]
    r = A.shape[1] // g
    Ntot = sum(Ns)
    dt = _compute_dtype(X)
    for t, n in ((G, "G"), (X, "X"), (Z, "Z"), (A, "A"), (B, "B")):
        _require_cuda(t, n, dt)
    if need_dx and dX is None:
        dX = torch.empty(M, K, dtype=dt, device=X.device)
    if need_dx:
        _require_cuda(dX, "dX", dt)
    if dA is None:
        dA = torch.empty(K, g * r, dtype=torch.float32, device=X.device)
    if dB is None:
        dB = torch.empty(r, Ntot, dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = torch.empty(max(qlora_grouped_workspace_bytes(M, K, Ns, r)[1], 256), dtype=torch.uint8,
                                device=X.device)
    _check(lib().qlora_grouped_bwd_dt(_COMPUTE[dt], M, K, g, Narr, r, G.data_ptr(), X.data_ptr(), Z.data_ptr(),
                                      Sarr, A.data_ptr(), B.data_ptr(), ctypes.c_float(c),
                                      dX.data_ptr() if need_dx else None, dA.data_ptr(), dB.data_ptr(),
                                      workspace.data_ptr(), workspace.numel(), _stream(stream)),
           "qlora_grouped_bwd_dt")
    return (dX if need_dx else None), dA, dB


NF4_AB_BF16, NF4_AB_F32, NF4_AB_F16 = 0, 1, 2


class _ComputeMap:
    """torch dtype -> NF4_COMPUTE_* code (torch is imported lazily)."""

    def __getitem__(self, dt):
        import torch
        return {torch.bfloat16: NF4_COMPUTE_BF16, torch.float16: NF4_COMPUTE_F16}[dt]


_COMPUTE = _ComputeMap()


def _compute_dtype(X):
    import torch
    if X.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"the compute type is bf16 or fp16, got {X.dtype}")
    return X.dtype


def qlora_merge(state: NF4State, A, B, c: float, K: int, N: int, out=None, stream=None):
    """W' = fl32(ŵ + c A B) as a K*N fp32 tensor (A: K x r, B: r x N, both
    bf16 or both fp32); pass it to nf4_quantize to re-quantize."""
    import torch
    r = A.shape[1]
    if A.dtype != B.dtype or A.dtype not in (torch.bfloat16, torch.float32, torch.float16):
        raise ValueError("A and B must both be bf16, both fp16 or both fp32")
    for t, n in ((A, "A"), (B, "B")):
        _require_cuda(t, n, A.dtype)
    if tuple(A.shape) != (K, r) or tuple(B.shape) != (r, N):
        raise ValueError("A must be K x r and B r x N")
    if out is None:
        out = torch.empty(K * N, dtype=torch.float32, device=A.device)
    st = state.c_struct()
    _check(lib().qlora_merge(K, N, r, ctypes.byref(st), A.data_ptr(), B.data_ptr(),
                             {torch.float32: NF4_AB_F32, torch.float16: NF4_AB_F16}.get(A.dtype, NF4_AB_BF16),
                             ctypes.c_float(c),
                             out.data_ptr(), _stream(stream)), "qlora_merge")
    return out


def qlora_merge_requantize(state: NF4State, A, B, c: float, K: int, N: int, stream=None):
    """Merge, then re-quantize: returns (new NF4State, device status word)."""
    return nf4_quantize(qlora_merge(state, A, B, c, K, N, stream=stream), stream=stream)


def qlora_sgd_step(A, B, dA, dB, lr: float, A_master=None, B_master=None, stream=None) -> None:
    """In-place SGD step on the bf16 or fp16 adapter (optionally through fp32 masters)."""
    import torch
    K, r = A.shape
    N = B.shape[1]
    pdt = _compute_dtype(A)
    for t, n, dt in ((A, "A", pdt), (B, "B", pdt), (dA, "dA", torch.float32),
                     (dB, "dB", torch.float32)):
        _require_cuda(t, n, dt)
    for m, n in ((A_master, "A_master"), (B_master, "B_master")):
        if m is not None:
            _require_cuda(m, n, torch.float32)
    _check(lib().qlora_sgd_step_dt(_COMPUTE[pdt], K, N, r, A.data_ptr(), B.data_ptr(), dA.data_ptr(),
                                   dB.data_ptr(), ctypes.c_float(lr), _ptr(A_master), _ptr(B_master),
                                   _stream(stream)), "qlora_sgd_step_dt")


def nf4_status_read(status, stream=None) -> int:
    v = ctypes.c_int32()
    _check(lib().nf4_status_read(status.data_ptr(), ctypes.byref(v), _stream(stream)), "nf4_status_read")
    return v.value


def qlora_workspace_bytes(M: int, K: int, N: int, r: int) -> tuple[int, int]:
    f, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().qlora_workspace_bytes(M, K, N, r, ctypes.byref(f), ctypes.byref(b)), "qlora_workspace_bytes")
    return f.value, b.value


def qlora_linear_fwd(X, state: NF4State, A, B, c: float, K: int, N: int, Y=None, Z=None,
                     workspace=None, stream=None, return_z: bool = True):
    """Y = X Ŵ + c (X A) B.  X: M x K, A: K x r, B: r x N, all bf16 or all fp16
    (the compute type).  Returns (Y, Z); with return_z=False and no Z given,
    Z stays in the workspace and (Y, None) is returned."""
    import torch
    M, r = X.shape[0], A.shape[1]
    dt = _compute_dtype(X)
    for t, n in ((X, "X"), (A, "A"), (B, "B")):
        _require_cuda(t, n, dt)
    if Y is None:
        Y = torch.empty(M, N, dtype=dt, device=X.device)
    if Z is None and return_z:
        Z = torch.empty(M, r, dtype=dt, device=X.device)
    if workspace is None:
        workspace = torch.empty(max(qlora_workspace_bytes(M, K, N, r)[0], 256), dtype=torch.uint8,
                                device=X.device)
    st = state.c_struct()
    _check(lib().qlora_linear_fwd_dt(_COMPUTE[dt], M, K, N, r, X.data_ptr(), ctypes.byref(st), A.data_ptr(),
                                     B.data_ptr(), float(c), Y.data_ptr(), _ptr(Z), workspace.data_ptr(),
                                     workspace.numel(), _stream(stream)), "qlora_linear_fwd_dt")
    return Y, Z


def qlora_linear_fwd_noalloc(X, state: NF4State, A, B, c: float, K: int, N: int, Y, Z=None, stream=None):
    """qlora_linear_fwd (bf16) with the library's own device scratch instead
    of a workspace: allocates nothing.  Y (and Z, if given) must be passed
    in.  Shapes whose forward workspace exceeds NF4_NOALLOC_SCRATCH_BYTES
    are rejected.  Returns (Y, Z)."""
    import torch
    M, r = X.shape[0], A.shape[1]
    for t, n in ((X, "X"), (A, "A"), (B, "B"), (Y, "Y")):
        _require_cuda(t, n, torch.bfloat16)
    if Z is not None:
        _require_cuda(Z, "Z", torch.bfloat16)
    st = state.c_struct()
    _check(lib().qlora_linear_fwd_noalloc(M, K, N, r, X.data_ptr(), ctypes.byref(st), A.data_ptr(), B.data_ptr(),
                                          float(c), Y.data_ptr(), _ptr(Z), _stream(stream)),
           "qlora_linear_fwd_noalloc")
    return Y, Z


def qlora_linear_bwd(G, X, Z, state: NF4State, A, B, c: float, K: int, N: int, need_dx: bool = True,
                     dX=None, dA=None, dB=None, workspace=None, stream=None):
    """dZ = c G Bᵀ, dA = Xᵀ dZ, dB = c Zᵀ G, dX = G Ŵᵀ + dZ Aᵀ.  Returns (dX, dA, dB).
    Z = None recomputes Z = X A in the workspace."""
    import torch
    M, r = X.shape[0], A.shape[1]
    dt = _compute_dtype(X)
    for t, n in ((G, "G"), (X, "X"), (Z, "Z"), (A, "A"), (B, "B")):
        if t is not None or n != "Z":
            _require_cuda(t, n, dt)
    if need_dx and dX is None:
        dX = torch.empty(M, K, dtype=dt, device=X.device)
    if dA is None:
        dA = torch.empty(K, r, dtype=torch.float32, device=X.device)
    if dB is None:
        dB = torch.empty(r, N, dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = torch.empty(max(qlora_workspace_bytes(M, K, N, r)[1], 256), dtype=torch.uint8,
                                device=X.device)
    st = state.c_struct()
    _check(lib().qlora_linear_bwd_dt(_COMPUTE[dt], M, K, N, r, G.data_ptr(), X.data_ptr(), _ptr(Z),
                                     ctypes.byref(st), A.data_ptr(), B.data_ptr(), float(c),
                                     _ptr(dX if need_dx else None), dA.data_ptr(), dB.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), _stream(stream)), "qlora_linear_bwd_dt")
    return (dX if need_dx else None), dA, dB


def qlora_timer_enable(kernel: str, enable: bool = True) -> None:
    _check(lib().qlora_timer_enable(KERNEL_IDS[kernel], int(enable)), "qlora_timer_enable")


def qlora_timer_read(kernel: str) -> tuple[float, int]:
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().qlora_timer_read(KERNEL_IDS[kernel], ctypes.byref(ms), ctypes.byref(n)), "qlora_timer_read")
    return ms.value, n.value
