"""ctypes binding of libtide_probe.so (include/tide_probe.h): occupancy and interference probes.

Measurement instruments only (GEMM-shaped and small spin workgroups that record where and when
they ran); the reduce-scatter and placement path never uses them.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
TIDE_PROBE_GEMM_SHAPED = 0
TIDE_PROBE_SMALL = 1
TIDE_PROBE_MIX_BOTH = 0
TIDE_PROBE_MIX_READS = 1
TIDE_PROBE_MIX_WRITES = 2
RECORD_BYTES = 32
_lib = None


class Rect(ctypes.Structure):
    """tide_probe_rect: `rows` rows of `width` bytes from src + i*src_pitch to dst + i*dst_pitch."""

    _fields_ = [("dst", ctypes.c_void_p), ("src", ctypes.c_void_p), ("dst_pitch", ctypes.c_int64),
                ("src_pitch", ctypes.c_int64), ("width", ctypes.c_int64), ("rows", ctypes.c_int64)]


def load_probe_library():
    global _lib
    if _lib is None:
        path = os.path.join(_PKG, "libtide_probe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m all_gather_placement_amd.build`")
        lib = ctypes.CDLL(path)
        from .build import PROBE_LIB, check_current

        check_current(PROBE_LIB, loaded=lib)
        lib.tide_probe_launch.restype = ctypes.c_int32
        lib.tide_probe_launch.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p]
        lib.tide_probe_mix.restype = ctypes.c_int32
        lib.tide_probe_mix.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
        lib.tide_probe_clock.restype = ctypes.c_int32
        lib.tide_probe_clock.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.tide_probe_stream_create_cu_mask.restype = ctypes.c_int32
        lib.tide_probe_stream_create_cu_mask.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
        lib.tide_probe_stream_destroy.restype = ctypes.c_int32
        lib.tide_probe_stream_destroy.argtypes = [ctypes.c_void_p]
        lib.tide_probe_wall_clock_khz.restype = ctypes.c_int64
        lib.tide_probe_wall_clock_khz.argtypes = []
        lib.tide_probe_dma_rect_copies.restype = ctypes.c_int32
        lib.tide_probe_dma_rect_copies.argtypes = [ctypes.c_int32, ctypes.POINTER(Rect), ctypes.c_int64,
                                                   ctypes.POINTER(ctypes.c_double)]
        _lib = lib
    return _lib


def probe_launch(num_wgs: int, shape: int, spin_ticks: int, records=None, stream=None):
    """records: a torch uint8/int64 cuda tensor of at least num_wgs * 32 bytes, or None."""
    lib = load_probe_library()
    if records is not None and records.numel() * records.element_size() < num_wgs * RECORD_BYTES:
        raise ValueError("records buffer too small")
    if stream is None:
        import torch

        stream = torch.cuda.current_stream()
    handle = stream if isinstance(stream, int) else stream.cuda_stream
    rc = lib.tide_probe_launch(int(num_wgs), int(shape), int(spin_ticks),
                               None if records is None else records.data_ptr(), handle)
    if rc != 0:
        raise RuntimeError(f"tide_probe_launch failed: {rc}")


def mix_launch(C: int, mode: int, src, dst, items: int, lds_bytes: int = 0, stream=None):
    """Launch the RS-shaped mix probe.  src: int64 cuda tensor of C contributor pointers (bf16, 1024*items
    each, 16-byte aligned); dst: fp32 cuda tensor of 1024*items elements, 16-byte aligned."""
    lib = load_probe_library()
    if dst.dtype.itemsize != 4 or dst.numel() < 1024 * items or not dst.is_cuda or dst.data_ptr() % 16:
        raise ValueError("dst must be a 16-byte-aligned 4-byte cuda tensor of at least 1024*items elements")
    if mode != TIDE_PROBE_MIX_WRITES and (src is None or src.numel() < C or not src.is_cuda):
        raise ValueError("src must be a cuda tensor of at least C pointers")
    if stream is None:
        import torch

        stream = torch.cuda.current_stream()
    handle = stream if isinstance(stream, int) else stream.cuda_stream
    rc = lib.tide_probe_mix(int(C), int(mode), None if src is None else src.data_ptr(), dst.data_ptr(), int(items),
                            int(lds_bytes), handle)
    if rc != 0:
        raise RuntimeError(f"tide_probe_mix failed: {rc}")


def clock_probe(spin_ticks: int, out, stream=None):
    """Launch the shader clock probe; out: a torch int64 cuda tensor of at least 4 elements."""
    lib = load_probe_library()
    if out.numel() * out.element_size() < 32 or not out.is_cuda:
        raise ValueError("out must be a cuda tensor of at least 32 bytes")
    if stream is None:
        import torch

        stream = torch.cuda.current_stream()
    handle = stream if isinstance(stream, int) else stream.cuda_stream
    rc = lib.tide_probe_clock(int(spin_ticks), out.data_ptr(), handle)
    if rc != 0:
        raise RuntimeError(f"tide_probe_clock failed: {rc}")


def clock_mhz(out_host, wall_khz: int) -> float:
    """Mean shader clock (MHz) from the probe's four values (a host sequence of 4 integers)."""
    w0, w1, c0, c1 = (int(x) & 0xFFFFFFFFFFFFFFFF for x in list(out_host)[:4])
    return (c1 - c0) / max(w1 - w0, 1) * wall_khz / 1e3


def cu_mask_stream(first_cu: int, n_cus: int):
    """A torch stream whose kernels may run only on CU-mask bits [first_cu, first_cu + n_cus).
    Returns (torch stream, handle); release the handle with destroy_stream once its work is done."""
    import torch

    h = ctypes.c_void_p()
    rc = load_probe_library().tide_probe_stream_create_cu_mask(int(first_cu), int(n_cus), ctypes.byref(h))
    if rc != 0:
        raise RuntimeError(f"tide_probe_stream_create_cu_mask({first_cu}, {n_cus}) failed: {rc}")
    return torch.cuda.ExternalStream(h.value), h.value


def destroy_stream(handle: int) -> None:
    rc = load_probe_library().tide_probe_stream_destroy(handle)
    if rc != 0:
        raise RuntimeError(f"tide_probe_stream_destroy failed: {rc}")


def wall_clock_khz() -> int:
    return int(load_probe_library().tide_probe_wall_clock_khz())


def decode(records_host):
    """numpy (n, 4) uint64 view of the records -> dict of arrays: start, end, xcc, se, sh, cu, cu_key."""
    import numpy as np

    r = np.asarray(records_host).reshape(-1, 4)
    hw = (r[:, 2] & 0xFFFFFFFF).astype(np.int64)
    xcc = ((r[:, 2] >> 32) & 0xF).astype(np.int64)
    cu = (hw >> 8) & 0xF
    sh = (hw >> 12) & 0x1
    se = (hw >> 13) & 0x3
    return {"start": r[:, 0].astype(np.int64), "end": r[:, 1].astype(np.int64), "xcc": xcc, "se": se, "sh": sh,
            "cu": cu, "cu_key": ((xcc * 4 + se) * 2 + sh) * 16 + cu}


def dma_rect_copies(rects, timeout_ms: int = 10000) -> float:
    """Run rectangular copies on the DMA engines (tide_probe_dma_rect_copies): `rects` is a sequence of
    (dst, src, dst_pitch, src_pitch, width, rows) with device addresses and byte sizes.  The copies
    are not stream-ordered: synchronise the device before the call.  Returns the host time from the
    first issue to the last completion, in microseconds."""
    lib = load_probe_library()
    arr = (Rect * max(len(rects), 1))(*[Rect(*r) for r in rects])
    us = ctypes.c_double()
    rc = lib.tide_probe_dma_rect_copies(len(rects), arr, int(timeout_ms), ctypes.byref(us))
    if rc != 0:
        raise RuntimeError(f"tide_probe_dma_rect_copies failed: {rc}")
    return us.value
