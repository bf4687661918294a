"""Binding of the measurement microkernels (``libgqa_peaks.so``, declared in
``include/gqa_peaks.h``): a bf16 MFMA-only loop and a streaming read, the
measured counterparts of the published bf16 matrix and HBM peaks.  Argument
marshalling only; raises if the library has not been built."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
PEAKS_LIB_PATH = os.path.join(_HERE, "libgqa_peaks.so")
_lib = None

# work per call, as the header states it
MFMA_FLOP_PER_WAVE_ITER = 8 * 32768


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PEAKS_LIB_PATH):
            raise ImportError(f"{PEAKS_LIB_PATH} is missing: build it with "
                              "`python -m transformer_attention_layer_amd.build`")
        L = ctypes.CDLL(PEAKS_LIB_PATH)
        L.gqa_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p]
        L.gqa_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p]
        L.gqa_peak_mfma_bf16.restype = ctypes.c_int
        L.gqa_peak_stream_read.restype = ctypes.c_int
        _lib = L
    return _lib


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def mfma_bf16(workgroups: int, iters: int, sink, stream=None) -> float:
    """Enqueue the MFMA loop; returns its FLOP count.  ``sink``: float32
    device tensor of workgroups * 256 entries."""
    if sink.numel() < workgroups * 256:
        raise ValueError("sink too small")
    r = lib().gqa_peak_mfma_bf16(workgroups, iters, sink.data_ptr(), _stream(stream))
    if r != 0:
        raise RuntimeError(f"gqa_peak_mfma_bf16 failed ({r})")
    return float(workgroups) * 4 * iters * MFMA_FLOP_PER_WAVE_ITER


def stream_read(buf, workgroups: int, sink, stream=None) -> int:
    """Enqueue the streaming read of ``buf`` (a device tensor whose byte size
    is a multiple of 32768); returns the bytes read.  ``sink``: int32 device
    tensor of workgroups * 256 entries."""
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() < workgroups * 256:
        raise ValueError("sink too small")
    r = lib().gqa_peak_stream_read(buf.data_ptr(), nbytes, workgroups, sink.data_ptr(),
                                   _stream(stream))
    if r != 0:
        raise RuntimeError(f"gqa_peak_stream_read failed ({r})")
    return nbytes
