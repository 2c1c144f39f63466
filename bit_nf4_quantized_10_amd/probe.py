"""Binding of libqlora_probe.so (include/qlora_read_probe.h): a plain
streaming read of a device buffer, timed by the benchmark as the device's
own read ceiling at the size of a memory-bound kernel's input."""
from __future__ import annotations

import ctypes
import os

PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora_probe.so")
C_FUNCTIONS = ["qlora_read_probe"]
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(f"{PROBE_PATH} is missing: build it with "
                               "`python -m bit_nf4_quantized_10_amd.build_lib`")
        # PyTorch brings its own HIP and HSA runtimes.  Loaded first, they
        # satisfy this library's libamdhip64 dependency, so the process holds
        # one HSA runtime; loaded the other way round, the process ends up
        # with two, and the second cannot reach the GPU.
        import torch  # noqa: F401
        L = ctypes.CDLL(PROBE_PATH)
        L.qlora_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
        L.qlora_read_probe.restype = ctypes.c_int
        _lib = L
    return _lib


def read_probe(buf, sink, grid: int = 4096, stream=None) -> None:
    """Stream every byte of the contiguous device tensor `buf` once
    (`sink`: a device int32/uint32 tensor of one element)."""
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    rc = lib().qlora_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), grid, sink.data_ptr(),
                                s.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"qlora_read_probe failed with code {rc}")
