"""Python binding of libbnn_calib.so (include/bnn_calib.h): rate probes for
the roofline fractions of the benchmark.  Not part of the product path.

Each probe enqueues one kernel on torch's current stream and returns the
per-block counter records (a ``(blocks, 4)`` int64 CUDA tensor: shader
cycles at start / end, wall clock ticks at start / end).  Raises if the
library is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libbnn_calib.so")

EXPORTED = ("bnn_calib_valu", "bnn_calib_mfma_fp4", "bnn_calib_mfma_fp4_pm1", "bnn_calib_read",
            "bnn_calib_wallclock_hz")

_lib = None


def library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is missing: run packed_xor_popcount_amd/build.py")
    lib = ctypes.CDLL(library_path)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.bnn_calib_valu.argtypes = [P, I64, I64, P]
    lib.bnn_calib_mfma_fp4.argtypes = [P, I64, I64, P]
    lib.bnn_calib_mfma_fp4_pm1.argtypes = [P, I64, I64, P]
    lib.bnn_calib_read.argtypes = [P, I64, P, I64, P]
    for n in ("bnn_calib_valu", "bnn_calib_mfma_fp4", "bnn_calib_mfma_fp4_pm1", "bnn_calib_read"):
        getattr(lib, n).restype = ctypes.c_int
    lib.bnn_calib_wallclock_hz.argtypes, lib.bnn_calib_wallclock_hz.restype = [], I64
    _lib = lib
    return lib


def _records(blocks: int, device) -> torch.Tensor:
    return torch.zeros(4 * blocks + 1, dtype=torch.int64, device=device)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _done(st: int, out: torch.Tensor, blocks: int, name: str) -> torch.Tensor:
    if st != 0:
        raise RuntimeError(f"{name}: status {st}")
    return out[: 4 * blocks].view(blocks, 4)


def valu(blocks: int, iters: int, device="cuda:0") -> torch.Tensor:
    """64 * iters VALU lane operations (xor, popcount) per thread."""
    out = _records(blocks, device)
    st = library().bnn_calib_valu(ctypes.c_void_p(out.data_ptr()), blocks, iters, _stream(device))
    return _done(st, out, blocks, "bnn_calib_valu")


def mfma_fp4(blocks: int, iters: int, device="cuda:0") -> torch.Tensor:
    """4 * iters FP4 32x32x64 MFMAs (131072 flops each) per wave, 4 waves per block."""
    out = _records(blocks, device)
    st = library().bnn_calib_mfma_fp4(ctypes.c_void_p(out.data_ptr()), blocks, iters,
                                      _stream(device))
    return _done(st, out, blocks, "bnn_calib_mfma_fp4")


def mfma_fp4_pm1(blocks: int, iters: int, device="cuda:0") -> torch.Tensor:
    """As mfma_fp4, with pseudo-random +-1 operands that change from one MFMA
    to the next."""
    out = _records(blocks, device)
    st = library().bnn_calib_mfma_fp4_pm1(ctypes.c_void_p(out.data_ptr()), blocks, iters,
                                          _stream(device))
    return _done(st, out, blocks, "bnn_calib_mfma_fp4_pm1")


def read(buf: torch.Tensor, blocks: int) -> torch.Tensor:
    """Read every byte of the contiguous CUDA tensor ``buf`` once."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous CUDA tensor")
    out = _records(blocks, buf.device)
    nbytes = buf.numel() * buf.element_size()
    st = library().bnn_calib_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                  ctypes.c_void_p(out.data_ptr()), blocks, _stream(buf.device))
    return _done(st, out, blocks, "bnn_calib_read")


def wallclock_hz() -> int:
    return int(library().bnn_calib_wallclock_hz())
