"""Achievable peaks of the chip (include/ttt_peaks.h), measured beside its
published ones: an HBM copy with 16-byte non-temporal accesses, a bf16
matrix-core issue loop and an fp32 vector (v_fma_f32) issue loop.  Thin ctypes binding plus the timing helpers that
``bench.py`` uses to state a roofline fraction against both.
"""
from __future__ import annotations

import ctypes

from . import _done, _ptr, _stream_handle, lib

PEAK_EXPORTS = ("ttt_peak_copy", "ttt_peak_mfma_bf16", "ttt_peak_mfma_bf16_flops", "ttt_peak_valu_f32",
                "ttt_peak_valu_f32_flops")


def _plib() -> ctypes.CDLL:
    L = lib()
    if not getattr(L, "_peaks_typed", False):
        vp = ctypes.c_void_p
        L.ttt_peak_copy.argtypes = [vp, vp, ctypes.c_int64, vp]
        L.ttt_peak_copy.restype = ctypes.c_int
        L.ttt_peak_mfma_bf16.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp]
        L.ttt_peak_mfma_bf16.restype = ctypes.c_int
        L.ttt_peak_mfma_bf16_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.ttt_peak_mfma_bf16_flops.restype = ctypes.c_int64
        L.ttt_peak_valu_f32.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp]
        L.ttt_peak_valu_f32.restype = ctypes.c_int
        L.ttt_peak_valu_f32_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.ttt_peak_valu_f32_flops.restype = ctypes.c_int64
        L._peaks_typed = True
    return L


def copy(src, dst, stream=None) -> None:
    """dst <- src (device tensors of the same byte size, a multiple of 16)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst differ in size")
    st = _plib().ttt_peak_copy(_ptr(src), _ptr(dst), n, _stream_handle(stream))
    _done(st, "ttt_peak_copy")


def mfma_bf16(out, blocks: int, iters: int, stream=None) -> None:
    """The matrix-core issue loop; out: float32 device tensor of blocks * 1024 elements."""
    if out.numel() < blocks * 1024:
        raise ValueError("out too small")
    st = _plib().ttt_peak_mfma_bf16(_ptr(out), int(blocks), int(iters), _stream_handle(stream))
    _done(st, "ttt_peak_mfma_bf16")


def mfma_bf16_flops(blocks: int, iters: int) -> int:
    return int(_plib().ttt_peak_mfma_bf16_flops(int(blocks), int(iters)))


def valu_f32(out, blocks: int, iters: int, stream=None) -> None:
    """The fp32 vector issue loop; out: float32 device tensor of blocks * 256 elements."""
    if out.numel() < blocks * 256:
        raise ValueError("out too small")
    st = _plib().ttt_peak_valu_f32(_ptr(out), int(blocks), int(iters), _stream_handle(stream))
    _done(st, "ttt_peak_valu_f32")


def valu_f32_flops(blocks: int, iters: int) -> int:
    return int(_plib().ttt_peak_valu_f32_flops(int(blocks), int(iters)))


def _time(fn, warmup: int, reps: int) -> float:
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps / 1e3  # seconds per call


def measure_hbm_copy(nbytes: int = 2 << 30, warmup: int = 10, reps: int = 20) -> float:
    """Sustained HBM bandwidth of the copy kernel, GB/s (bytes read + written); 2 GiB
    each way by default, so the 256 MB last-level cache holds a negligible share."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    sec = _time(lambda: copy(src, dst), warmup, reps)
    del src, dst
    return 2 * nbytes / sec / 1e9


def measure_mfma_bf16(blocks: int = 512, iters: int = 20000, warmup: int = 2, reps: int = 5) -> float:
    """Sustained dense bf16 matrix-core rate of the issue loop, TFLOP/s."""
    import torch

    out = torch.empty(blocks * 1024, dtype=torch.float32, device="cuda:0")
    sec = _time(lambda: mfma_bf16(out, blocks, iters), warmup, reps)
    return mfma_bf16_flops(blocks, iters) / sec / 1e12


def measure_valu_f32(blocks: int = 2048, iters: int = 50000, warmup: int = 2, reps: int = 5) -> float:
    """Sustained unpacked fp32 vector-FMA rate of the issue loop, TFLOP/s."""
    import torch

    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    sec = _time(lambda: valu_f32(out, blocks, iters), warmup, reps)
    return valu_f32_flops(blocks, iters) / sec / 1e12
