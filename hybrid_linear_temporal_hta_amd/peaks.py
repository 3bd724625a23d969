"""ctypes binding of libhta_peaks.so (include/hta_peaks.h): the MFMA issue loop,
the HBM copy, and the global->LDS load and LDS read loops whose rates the
benchmark reports beside the published peaks. Argument marshalling only; the
library must be built (it raises otherwise)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhta_peaks.so")
EXPORTED = ("hta_peak_mfma", "hta_peak_mfma_chains", "hta_peak_copy", "hta_peak_lds_dma",
            "hta_peak_lds_read")
MFMA_FLOP = 2 * 32 * 32 * 16          # one v_mfma_f32_32x32x16_bf16 per wave
WAVES_PER_BLOCK = 4

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python -m "
                               "hybrid_linear_temporal_hta_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i = ctypes.c_void_p, ctypes.c_int
        L.hta_peak_mfma.restype = i
        L.hta_peak_mfma.argtypes = [i, i, vp, vp]
        L.hta_peak_mfma_chains.restype = i
        L.hta_peak_mfma_chains.argtypes = []
        L.hta_peak_copy.restype = i
        L.hta_peak_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        L.hta_peak_lds_dma.restype = i
        L.hta_peak_lds_dma.argtypes = [vp, ctypes.c_size_t, i, i, i, vp]
        L.hta_peak_lds_read.restype = i
        L.hta_peak_lds_read.argtypes = [i, i, i, vp, vp]
        _lib = L
    return _lib


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def mfma_flop(blocks: int, iters: int) -> float:
    return float(blocks) * WAVES_PER_BLOCK * iters * lib().hta_peak_mfma_chains() * MFMA_FLOP


def mfma(blocks: int, iters: int, sink, stream=None) -> None:
    st = lib().hta_peak_mfma(int(blocks), int(iters), ctypes.c_void_p(sink.data_ptr()),
                             _stream(stream))
    if st != 0:
        raise RuntimeError(f"hta_peak_mfma: status {st}")


def copy(src, dst, stream=None) -> None:
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    st = lib().hta_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n,
                             _stream(stream))
    if st != 0:
        raise RuntimeError(f"hta_peak_copy: status {st}")


def lds_dma_bytes(blocks: int, iters: int) -> float:
    return float(blocks) * WAVES_PER_BLOCK * iters * 8 * 1024


def lds_dma(src, window_bytes: int, blocks: int, iters: int, pattern: int, stream=None) -> None:
    if window_bytes > src.numel() * src.element_size():
        raise ValueError("window larger than src")
    st = lib().hta_peak_lds_dma(ctypes.c_void_p(src.data_ptr()), int(window_bytes), int(blocks),
                                int(iters), int(pattern), _stream(stream))
    if st != 0:
        raise RuntimeError(f"hta_peak_lds_dma: status {st}")


def lds_read_bytes(blocks: int, iters: int, transposed: bool) -> float:
    return float(blocks) * WAVES_PER_BLOCK * iters * 8 * (512 if transposed else 1024)


def lds_read(blocks: int, iters: int, transposed: bool, sink, stream=None) -> None:
    st = lib().hta_peak_lds_read(int(blocks), int(iters), int(bool(transposed)),
                                 ctypes.c_void_p(sink.data_ptr()), _stream(stream))
    if st != 0:
        raise RuntimeError(f"hta_peak_lds_read: status {st}")
