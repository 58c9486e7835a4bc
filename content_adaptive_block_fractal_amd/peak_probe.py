"""The benchmark's measurement aid, libcabf_probe.so: a dense bf16 matrix-core
loop whose time gives the rate the chip sustains under load, to set beside the
published peak. It is not part of the attention path and not in libcabf's ABI.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcabf_probe.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python content_adaptive_block_fractal_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        lib.probe_mfma_peak.restype = ctypes.c_int
        lib.probe_mfma_peak.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]
        _lib = lib
    return _lib


def mfma_peak(workgroups: int, iters: int, out: torch.Tensor):
    """workgroups x 256 threads, each wave iters x 8 products of 32x32x16 bf16
    (262144 * iters flops per wave); out: float32 device tensor of workgroups * 256
    values (without meaning). Launched on torch's current stream."""
    if not out.is_cuda or out.dtype != torch.float32 or out.numel() != workgroups * 256:
        raise ValueError("out must be a float32 device tensor of workgroups * 256 elements")
    stream = ctypes.c_void_p(torch.cuda.current_stream(out.device).cuda_stream)
    st = _load().probe_mfma_peak(int(workgroups), int(iters), ctypes.c_void_p(out.data_ptr()),
                                 stream)
    if st != 0:
        raise RuntimeError(f"probe_mfma_peak failed: {st}")
