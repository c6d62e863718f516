"""Python binding of libfa16measure.so (include/fa16measure.h): measurement
aids for the benchmark, not part of the attention method.

Argument marshalling only; raises if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa16measure.so")
_lib = None

# Every symbol include/fa16measure.h declares.
EXPORTS = ("fa_mfma_ceiling",)
FAM_OK, FAM_ERR_NULL, FAM_ERR_SHAPE = 0, 1, 2
MFMA_CEILING_OUT = 512 * 256  # FP32 values fa_mfma_ceiling writes


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m fp16_attention_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.fa_mfma_ceiling.restype = ctypes.c_int
        lib.fa_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def mfma_ceiling_flop(iters: int) -> float:
    """FLOP of one fa_mfma_ceiling launch."""
    return 512.0 * 4 * iters * 4 * 32768


def mfma_ceiling(out, iters: int):
    """Launch the FP16 MFMA rate kernel on out's stream; out: CUDA float32
    tensor of at least MFMA_CEILING_OUT elements."""
    import torch
    if out.dtype != torch.float32 or out.numel() < MFMA_CEILING_OUT or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of MFMA_CEILING_OUT elements")
    if not out.is_cuda:
        raise ValueError("out must be a CUDA (HIP) tensor")
    rc = load().fa_mfma_ceiling(int(iters), out.data_ptr(), torch.cuda.current_stream(out.device).cuda_stream)
    if rc != FAM_OK:
        raise RuntimeError(f"fa_mfma_ceiling failed (code {rc})")
    return out
