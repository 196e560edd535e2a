"""packed_xor_popcount_amd -- Python binding of libbnn.so (include/bnn.h).

Packed binary (+1/-1) matrix products on MI355X (gfx950): sign projection and
packing along K, and <x, w> = K - 2 * popcount(x XOR w) with int32,
alpha-scaled fp32 or sign -> repack outputs ("Binary Math Effectiveness --
why / how / when", section 1).

This module only marshals arguments: it checks tensor devices, dtypes and
shapes, allocates outputs with PyTorch (device memory is PyTorch's; the
library allocates nothing), and passes raw device pointers and the current
HIP stream to the C entry points of the same names.  Every step of the
computation runs in the HIP kernels of libbnn.so; there is no CPU path.  If
libbnn.so is missing this module raises instead of falling back.

Packed matrices are ``torch.int64`` tensors of shape ``(rows, words(K))``
holding the uint64 words bit for bit (bit k%64 of word k/64 is element k,
least significant bit first; bit 1 means -1).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BnnError", "EPI_I32", "EPI_SCALED", "EPI_REPACK", "ALGO_AUTO", "ALGO_GEMV", "ALGO_TILED",
    "ALGO_MFMA",
    "library", "library_path", "words", "pack_signs", "gemm_u64", "gemm_u64_scaled",
    "gemm_sign_repack", "gemm_sign_repack_thr", "flip_words", "gemm_signw_bf16", "chain3",
    "gemm_ex", "gemv_act", "version",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libbnn.so")

BNN_FP32, BNN_BF16 = 0, 1
EPI_I32, EPI_SCALED, EPI_REPACK = 0, 1, 2
ALGO_AUTO, ALGO_GEMV, ALGO_TILED, ALGO_MFMA = 0, 1, 2, 3

EXPORTED = ("bnn_words", "bnn_status_str", "bnn_version", "bnn_pack_signs", "bnn_gemm_u64",
            "bnn_gemm_u64_scaled", "bnn_gemm_sign_repack", "bnn_gemm_ex", "bnn_gemv_act",
            "bnn_gemm_sign_repack_thr", "bnn_gemm_signw_bf16", "bnn_chain3")


class BnnError(RuntimeError):
    """A non-zero bnn_status returned by libbnn.so."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_status_str(status)} (status {status})")


_lib = None


def library():
    """The loaded libbnn.so (built in-tree first if it does not exist yet)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(library_path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.bnn_words.argtypes, lib.bnn_words.restype = [I64], I64
    lib.bnn_status_str.argtypes, lib.bnn_status_str.restype = [I], ctypes.c_char_p
    lib.bnn_version.argtypes, lib.bnn_version.restype = [], ctypes.c_char_p
    lib.bnn_pack_signs.argtypes = [P, I, I64, I64, I64, P, P]
    lib.bnn_gemm_u64.argtypes = [P, P, P, I64, I64, I64, P]
    lib.bnn_gemm_u64_scaled.argtypes = [P, P, P, P, I64, I64, I64, P]
    lib.bnn_gemm_sign_repack.argtypes = [P, P, P, I64, I64, I64, P]
    lib.bnn_gemm_ex.argtypes = [P, P, P, P, I64, I64, I64, I, I, P]
    lib.bnn_gemv_act.argtypes = [P, I, I64, P, P, P, I64, I64, I64, I, P]
    lib.bnn_gemm_sign_repack_thr.argtypes = [P, P, P, P, P, I64, I64, I64, I, P]
    lib.bnn_gemm_signw_bf16.argtypes = [P, I64, P, P, P, I64, I64, I64, I, P]
    lib.bnn_chain3.argtypes = [P, I, I64, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P]
    for name in ("bnn_pack_signs", "bnn_gemm_u64", "bnn_gemm_u64_scaled", "bnn_gemm_sign_repack",
                 "bnn_gemm_ex", "bnn_gemv_act", "bnn_gemm_sign_repack_thr", "bnn_gemm_signw_bf16",
                 "bnn_chain3"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _status_str(status: int) -> str:
    return library().bnn_status_str(int(status)).decode()


def version() -> str:
    return library().bnn_version().decode()


def words(k: int) -> int:
    """ceil(k/64): 64-bit words per packed row of k logical values."""
    return int(library().bnn_words(int(k)))


def _check(status: int, where: str) -> None:
    if status != 0:
        raise BnnError(status, where)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(name: str, t: torch.Tensor) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")


def _packed(name: str, t: torch.Tensor, k: int) -> int:
    _need_cuda(name, t)
    if t.dtype != torch.int64 or t.dim() != 2 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous 2-D int64 tensor of packed words")
    if t.shape[1] != words(k):
        raise ValueError(f"{name} has {t.shape[1]} words per row, K={k} needs {words(k)}")
    return t.shape[0]


def pack_signs(src: torch.Tensor, k: int | None = None, out: torch.Tensor | None = None):
    """Sign-project and pack a 2-D fp32 or bf16 CUDA tensor along its last
    dimension (the first ``k`` columns, default all).  Rows may be strided
    (``src.stride(1)`` must be 1).  Returns int64 ``(rows, words(k))``."""
    _need_cuda("src", src)
    if src.dim() != 2 or (src.shape[1] > 1 and src.stride(1) != 1):
        raise ValueError("src must be 2-D with unit stride along its last dimension")
    if src.dtype == torch.float32:
        dt = BNN_FP32
    elif src.dtype == torch.bfloat16:
        dt = BNN_BF16
    else:
        raise TypeError("src must be float32 or bfloat16")
    rows, cols = src.shape
    k = cols if k is None else int(k)
    ld = src.stride(0) if rows > 1 else max(cols, 1)
    if out is None:
        out = torch.empty((rows, words(k)), dtype=torch.int64, device=src.device)
    else:
        _packed("out", out, k)
    st = library().bnn_pack_signs(_ptr(src), dt, rows, k, ld, _ptr(out), _stream(src))
    _check(st, "bnn_pack_signs")
    return out


def gemm_ex(xp: torch.Tensor, wp: torch.Tensor, K: int, epilogue: int = EPI_I32,
            algo: int = ALGO_AUTO, alpha: torch.Tensor | None = None,
            out: torch.Tensor | None = None):
    """General packed product (bnn_gemm_ex): int32 (EPI_I32), alpha-scaled
    fp32 (EPI_SCALED) or packed signs (EPI_REPACK), with an explicit kernel
    family (ALGO_AUTO, ALGO_GEMV, ALGO_TILED, ALGO_MFMA)."""
    M = _packed("xp", xp, K)
    N = _packed("wp", wp, K)
    if wp.device != xp.device:
        raise ValueError("xp and wp must be on the same device")
    if epilogue == EPI_SCALED:
        _need_cuda("alpha", alpha)
        if alpha.dtype != torch.float32 or alpha.shape != (N,) or not alpha.is_contiguous():
            raise ValueError("alpha must be a contiguous float32 tensor of shape (N,)")
    out = _out_for(epilogue, M, N, xp.device, out)
    st = library().bnn_gemm_ex(_ptr(xp), _ptr(wp), _ptr(alpha) if epilogue == EPI_SCALED else None,
                               _ptr(out), M, N, int(K), int(epilogue), int(algo), _stream(xp))
    _check(st, "bnn_gemm_ex")
    return out


def _out_for(epilogue: int, M: int, N: int, device, out):
    if epilogue == EPI_I32:
        shape, dtype = (M, N), torch.int32
    elif epilogue == EPI_SCALED:
        shape, dtype = (M, N), torch.float32
    elif epilogue == EPI_REPACK:
        shape, dtype = (M, words(N)), torch.int64
    else:
        raise ValueError(f"unknown epilogue {epilogue}")
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(out.shape) != shape or out.dtype != dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {dtype} tensor of shape {shape}")
    return out


def gemv_act(x: torch.Tensor, wp: torch.Tensor, K: int | None = None, epilogue: int = EPI_I32,
             alpha: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """Product of real-valued activation rows ``x`` (fp32 or bf16, 2-D, unit
    stride along the last dimension; the first ``K`` columns are used) with
    packed weights ``wp``; the kernel packs ``x`` itself (bnn_gemv_act).
    Meant for small M (batch-1 decode)."""
    _need_cuda("x", x)
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be 2-D with unit stride along its last dimension")
    if x.dtype == torch.float32:
        dt = BNN_FP32
    elif x.dtype == torch.bfloat16:
        dt = BNN_BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    M, cols = x.shape
    K = cols if K is None else int(K)
    N = _packed("wp", wp, K)
    if epilogue == EPI_SCALED:
        _need_cuda("alpha", alpha)
        if alpha.dtype != torch.float32 or alpha.shape != (N,) or not alpha.is_contiguous():
            raise ValueError("alpha must be a contiguous float32 tensor of shape (N,)")
    out = _out_for(epilogue, M, N, x.device, out)
    ldx = x.stride(0) if M > 1 else max(cols, 1)
    st = library().bnn_gemv_act(_ptr(x), dt, ldx, _ptr(wp),
                                _ptr(alpha) if epilogue == EPI_SCALED else None, _ptr(out),
                                M, N, K, int(epilogue), _stream(x))
    _check(st, "bnn_gemv_act")
    return out


def _named(name: str, xp, wp, K, epilogue: int, alpha, out):
    """Marshal one of the three named products (same checks as gemm_ex) and
    call its own C entry point."""
    M = _packed("xp", xp, K)
    N = _packed("wp", wp, K)
    if wp.device != xp.device:
        raise ValueError("xp and wp must be on the same device")
    if epilogue == EPI_SCALED:
        _need_cuda("alpha", alpha)
        if alpha.dtype != torch.float32 or alpha.shape != (N,) or not alpha.is_contiguous():
            raise ValueError("alpha must be a contiguous float32 tensor of shape (N,)")
    out = _out_for(epilogue, M, N, xp.device, out)
    fn = getattr(library(), name)
    if epilogue == EPI_SCALED:
        st = fn(_ptr(xp), _ptr(wp), _ptr(alpha), _ptr(out), M, N, int(K), _stream(xp))
    else:
        st = fn(_ptr(xp), _ptr(wp), _ptr(out), M, N, int(K), _stream(xp))
    _check(st, name)
    return out


def gemm_u64(xp, wp, K, out=None):
    """int32 ``(M, N)``: ``<x_m, w_n> = K - 2 * popcount(x_m XOR w_n)`` (bnn_gemm_u64)."""
    return _named("bnn_gemm_u64", xp, wp, K, EPI_I32, None, out)


def gemm_u64_scaled(xp, wp, alpha, K, out=None):
    """fp32 ``(M, N)``: ``(float)<x_m, w_n> * alpha[n]`` (bnn_gemm_u64_scaled)."""
    return _named("bnn_gemm_u64_scaled", xp, wp, K, EPI_SCALED, alpha, out)


def gemm_sign_repack(xp, wp, K, out=None):
    """int64 ``(M, words(N))``: projected signs of ``<x_m, w_n>`` packed along N
    (bnn_gemm_sign_repack)."""
    return _named("bnn_gemm_sign_repack", xp, wp, K, EPI_REPACK, None, out)


def gemm_sign_repack_thr(xp, wp, thr, K, flip=None, algo=ALGO_AUTO, out=None):
    """int64 ``(M, words(N))``: bit n of row m is 1 when ``<x_m, w_n> <= thr[n]``,
    inverted where bit n of the packed ``flip`` mask is 1
    (bnn_gemm_sign_repack_thr; the folded form of a BatchNorm after a binary
    layer, see ``fold.bn_fold``).  ``thr`` is a contiguous int32 CUDA tensor
    ``(N,)``; ``flip`` is None or a contiguous int64 CUDA tensor
    ``(words(N),)`` (``flip_words`` builds one from per-channel flags)."""
    M = _packed("xp", xp, K)
    N = _packed("wp", wp, K)
    if wp.device != xp.device:
        raise ValueError("xp and wp must be on the same device")
    _need_cuda("thr", thr)
    if thr.dtype != torch.int32 or tuple(thr.shape) != (N,) or not thr.is_contiguous():
        raise ValueError("thr must be a contiguous int32 tensor of shape (N,)")
    if flip is not None:
        _need_cuda("flip", flip)
        if (flip.dtype != torch.int64 or tuple(flip.shape) != (words(N),)
                or not flip.is_contiguous()):
            raise ValueError("flip must be a contiguous int64 tensor of shape (words(N),)")
    out = _out_for(EPI_REPACK, M, N, xp.device, out)
    st = library().bnn_gemm_sign_repack_thr(_ptr(xp), _ptr(wp), _ptr(thr), _ptr(flip), _ptr(out),
                                            M, N, int(K), int(algo), _stream(xp))
    _check(st, "bnn_gemm_sign_repack_thr")
    return out


def flip_words(flags: torch.Tensor) -> torch.Tensor:
    """Packed flip mask ``(words(N),)`` from N per-channel flags on a CUDA
    device (non-zero = flip), packed by the library's sign packer: a flag
    maps to -1 (bit 1), no flag to +1 (bit 0)."""
    _need_cuda("flags", flags)
    if flags.dim() != 1:
        raise ValueError("flags must be 1-D")
    signs = torch.where(flags != 0, -1.0, 1.0).to(torch.float32).reshape(1, -1)
    return pack_signs(signs)[0]


def gemm_signw_bf16(x, wp, K=None, alpha=None, algo=ALGO_AUTO, out=None):
    """fp32 ``(M, N)``: ``alpha[n] * sum_k x[m, k] * w_n[k]`` for real-valued
    bf16 activations ``x`` (2-D CUDA tensor, unit stride along the last
    dimension; the first ``K`` columns are used) and packed sign weights
    ``wp`` (bnn_gemm_signw_bf16).  ``alpha`` is None (no scale) or a
    contiguous float32 ``(N,)``; ``algo`` is ALGO_AUTO, ALGO_GEMV or ALGO_MFMA."""
    _need_cuda("x", x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be 2-D with unit stride along its last dimension")
    M, cols = x.shape
    K = cols if K is None else int(K)
    N = _packed("wp", wp, K)
    if alpha is not None:
        _need_cuda("alpha", alpha)
        if alpha.dtype != torch.float32 or alpha.shape != (N,) or not alpha.is_contiguous():
            raise ValueError("alpha must be a contiguous float32 tensor of shape (N,)")
    out = _out_for(EPI_SCALED, M, N, x.device, out)
    ldx = x.stride(0) if M > 1 else max(cols, 1)
    st = library().bnn_gemm_signw_bf16(_ptr(x), ldx, _ptr(wp), _ptr(alpha), _ptr(out), M, N, K,
                                       int(algo), _stream(x))
    _check(st, "bnn_gemm_signw_bf16")
    return out


def chain3(x, w1, w2, w3, alpha3=None, out=None, thr1=None, flip1=None, thr2=None, flip2=None):
    """fp32 ``(M, N3)``: three chained binary layers in one launch
    (bnn_chain3).  ``x`` is a 2-D fp32 or bf16 CUDA tensor (unit stride along
    its last dimension, K0 columns); ``w1``, ``w2``, ``w3`` are packed weights
    ``(N1, words(K0))``, ``(N2, words(N1))``, ``(N3, words(N2))``; ``alpha3`` is
    None or a contiguous float32 ``(N3,)``.  ``thr1``/``flip1`` and
    ``thr2``/``flip2`` optionally make the hidden layers threshold repacks
    (as gemm_sign_repack_thr).  Equal, bit for bit, to pack_signs ->
    gemm_sign_repack(_thr) -> gemm_sign_repack(_thr) -> gemm_u64_scaled."""
    _need_cuda("x", x)
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be 2-D with unit stride along its last dimension")
    if x.dtype == torch.float32:
        dt = BNN_FP32
    elif x.dtype == torch.bfloat16:
        dt = BNN_BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    M, K0 = x.shape
    N1 = _packed("w1", w1, K0)
    N2 = _packed("w2", w2, N1)
    N3 = _packed("w3", w3, N2)
    if alpha3 is not None:
        _need_cuda("alpha3", alpha3)
        if alpha3.dtype != torch.float32 or alpha3.shape != (N3,) or not alpha3.is_contiguous():
            raise ValueError("alpha3 must be a contiguous float32 tensor of shape (N3,)")
    for name, t, n in (("thr1", thr1, N1), ("thr2", thr2, N2)):
        if t is not None:
            _need_cuda(name, t)
            if t.dtype != torch.int32 or tuple(t.shape) != (n,) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 tensor of shape ({n},)")
    for name, f, n in (("flip1", flip1, N1), ("flip2", flip2, N2)):
        if f is not None:
            _need_cuda(name, f)
            if f.dtype != torch.int64 or tuple(f.shape) != (words(n),) or not f.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int64 tensor of shape ({words(n)},)")
    out = _out_for(EPI_SCALED, M, N3, x.device, out)
    ldx = x.stride(0) if M > 1 else max(K0, 1)
    st = library().bnn_chain3(_ptr(x), dt, ldx, _ptr(w1), _ptr(thr1), _ptr(flip1), _ptr(w2),
                              _ptr(thr2), _ptr(flip2), _ptr(w3), _ptr(alpha3), _ptr(out), M, K0, N1,
                              N2, N3, _stream(x))
    _check(st, "bnn_chain3")
    return out
