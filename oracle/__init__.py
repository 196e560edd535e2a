"""Plain CPU oracle for packed binary (+1/-1) matrix products.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  It shares no code
with the HIP library (``packed_xor_popcount_amd``) and never imports it.

The arithmetic lives in ``bnn_oracle.c`` (plain C, compiled with gcc, no
fast-math, no FMA contraction).  This module only marshals numpy arrays.
What each function computes, and the page passages it follows, is stated in
``bnn_oracle.c``:

* "Binary Math Effectiveness -- why / how / when", section 1 "The core
  identity": the encoding table (bit 0 = +1, bit 1 = -1), the dot product of
  two +-1 vectors, and the edge-case table (padding, n = 0, alpha = 0, the
  projection of non-+-1 inputs);
* the same page, section 2.1: ceil(K/64) words per row.

Packed matrices are numpy ``uint64`` arrays of shape ``(rows, words(K))``;
bf16 inputs are numpy ``uint16`` arrays of raw bit patterns.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(identity, brute force, special cases, padding, projection table, library
witness, scaled closed form, repack composition, worked examples, threshold
repack, real-activation product).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bnn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libbnn_oracle.so")

GCC_CMD = [
    "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
    _SRC, "-o", _LIB_PATH,
]

_lib = None


def build_lib() -> str:
    """Compile the oracle shared library (plain gcc)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build_lib()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_words.argtypes = [I64]
    lib.oracle_words.restype = I64
    lib.oracle_sign_f32.argtypes = [ctypes.c_float]
    lib.oracle_sign_f32.restype = ctypes.c_int
    lib.oracle_sign_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_sign_bf16.restype = ctypes.c_int
    lib.oracle_pack_f32.argtypes = [P, I64, I64, I64, P]
    lib.oracle_pack_bf16.argtypes = [P, I64, I64, I64, P]
    lib.oracle_unpack.argtypes = [P, I64, I64, P]
    lib.oracle_gemm_i32.argtypes = [P, P, I64, I64, I64, P, ctypes.c_int]
    lib.oracle_gemm_scaled.argtypes = [P, P, P, I64, I64, I64, P, ctypes.c_int]
    lib.oracle_sign_repack.argtypes = [P, P, I64, I64, I64, P, ctypes.c_int]
    lib.oracle_dot_pairs.argtypes = [P, P, I64, P, P, I64, P]
    lib.oracle_sign_repack_thr.argtypes = [P, P, P, P, I64, I64, I64, P, ctypes.c_int]
    lib.oracle_dot_signw_bf16.argtypes = [P, I64, P, I64, I64, I64, P, ctypes.c_int]
    for name in ("oracle_pack_f32", "oracle_pack_bf16", "oracle_unpack", "oracle_gemm_i32",
                 "oracle_gemm_scaled", "oracle_sign_repack", "oracle_dot_pairs",
                 "oracle_sign_repack_thr", "oracle_dot_signw_bf16"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def words(k: int) -> int:
    """ceil(k/64): 64-bit words per packed row of k logical values."""
    return int(_load().oracle_words(int(k)))


def sign_f32(v: float) -> int:
    """+1 if v > 0 else -1 (zeros and NaN project to -1)."""
    return int(_load().oracle_sign_f32(float(v)))


def sign_bf16(bits: int) -> int:
    """Projection of a bf16 value given as its 16-bit pattern."""
    return int(_load().oracle_sign_bf16(int(bits) & 0xFFFF))


def pack(src: np.ndarray, k: int | None = None) -> np.ndarray:
    """Sign-project and pack a 2-D float32 array, or a uint16 array of bf16
    bit patterns, along its last axis.  Returns uint64 ``(rows, words(k))``."""
    lib = _load()
    src = np.asarray(src)
    if src.ndim != 2:
        raise ValueError("pack expects a 2-D array")
    rows, ld = src.shape
    k = ld if k is None else int(k)
    if k > ld:
        raise ValueError("k larger than the row length")
    if src.dtype == np.float32:
        fn = lib.oracle_pack_f32
    elif src.dtype == np.uint16:
        fn = lib.oracle_pack_bf16
    else:
        raise TypeError("pack expects float32 or uint16 (bf16 bits)")
    src = np.ascontiguousarray(src)
    out = np.zeros((rows, words(k)), dtype=np.uint64)
    if rows and k:
        fn(_ptr(src), rows, k, ld, _ptr(out))
    return out


def unpack(p: np.ndarray, k: int) -> np.ndarray:
    """Packed ``(rows, words(k))`` -> int8 ``(rows, k)`` of +1/-1."""
    p = np.ascontiguousarray(p, dtype=np.uint64)
    rows = p.shape[0]
    out = np.zeros((rows, k), dtype=np.int8)
    if rows and k:
        _load().oracle_unpack(_ptr(p), rows, k, _ptr(out))
    return out


def _check_packed(xp: np.ndarray, wp: np.ndarray, k: int):
    xp = np.ascontiguousarray(xp, dtype=np.uint64)
    wp = np.ascontiguousarray(wp, dtype=np.uint64)
    kw = words(k)
    if xp.ndim != 2 or wp.ndim != 2 or xp.shape[1] != kw or wp.shape[1] != kw:
        raise ValueError(f"packed operands must be (rows, {kw}) for K={k}")
    return xp, wp


def gemm_i32(xp: np.ndarray, wp: np.ndarray, k: int, nthreads: int = 0) -> np.ndarray:
    """int32 ``(M, N)``: ``Y[m, n] = <x_m, w_n>`` over the K logical elements."""
    xp, wp = _check_packed(xp, wp, k)
    M, N = xp.shape[0], wp.shape[0]
    y = np.zeros((M, N), dtype=np.int32)
    if M and N:
        _load().oracle_gemm_i32(_ptr(xp), _ptr(wp), M, N, k, _ptr(y), nthreads)
    return y


def gemm_scaled(xp: np.ndarray, wp: np.ndarray, alpha: np.ndarray, k: int,
                nthreads: int = 0) -> np.ndarray:
    """float32 ``(M, N)``: ``(float)<x_m, w_n> * alpha[n]``, one fp32 multiply."""
    xp, wp = _check_packed(xp, wp, k)
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    M, N = xp.shape[0], wp.shape[0]
    if alpha.shape != (N,):
        raise ValueError("alpha must have one value per output channel")
    y = np.zeros((M, N), dtype=np.float32)
    if M and N:
        _load().oracle_gemm_scaled(_ptr(xp), _ptr(wp), _ptr(alpha), M, N, k, _ptr(y), nthreads)
    return y


def sign_repack(xp: np.ndarray, wp: np.ndarray, k: int, nthreads: int = 0) -> np.ndarray:
    """uint64 ``(M, words(N))``: the projected signs of ``<x_m, w_n>`` packed
    along N (dot <= 0 -> bit 1), ready as the next binary layer's input."""
    xp, wp = _check_packed(xp, wp, k)
    M, N = xp.shape[0], wp.shape[0]
    y = np.zeros((M, words(N)), dtype=np.uint64)
    if M and N:
        _load().oracle_sign_repack(_ptr(xp), _ptr(wp), M, N, k, _ptr(y), nthreads)
    return y


def sign_repack_thr(xp: np.ndarray, wp: np.ndarray, thr: np.ndarray, k: int, flip=None,
                    nthreads: int = 0) -> np.ndarray:
    """uint64 ``(M, words(N))``: bit n of row m is 1 when ``<x_m, w_n> <= thr[n]``,
    inverted where ``flip[n]`` is non-zero (the folded form of a BatchNorm
    between binary layers)."""
    xp, wp = _check_packed(xp, wp, k)
    M, N = xp.shape[0], wp.shape[0]
    thr = np.ascontiguousarray(thr, dtype=np.int32)
    if thr.shape != (N,):
        raise ValueError("thr must have one value per output channel")
    fl = None if flip is None else np.ascontiguousarray(flip, dtype=np.uint8)
    if fl is not None and fl.shape != (N,):
        raise ValueError("flip must have one value per output channel")
    y = np.zeros((M, words(N)), dtype=np.uint64)
    if M and N:
        _load().oracle_sign_repack_thr(_ptr(xp), _ptr(wp), _ptr(thr),
                                       None if fl is None else _ptr(fl), M, N, k, _ptr(y), nthreads)
    return y


def dot_signw_bf16(x_bits: np.ndarray, wp: np.ndarray, k: int | None = None,
                   nthreads: int = 0) -> np.ndarray:
    """float64 ``(M, N)``: ``sum_k x[m, k] * w_n[k]`` for real-valued bf16
    activations (``uint16`` bit patterns, ``(M, >= k)``) and packed sign
    weights ``wp`` ``(N, words(k))``, summed in k order in double."""
    x_bits = np.asarray(x_bits)
    if x_bits.dtype != np.uint16 or x_bits.ndim != 2:
        raise TypeError("x_bits must be a 2-D uint16 array of bf16 bit patterns")
    M, ld = x_bits.shape
    k = ld if k is None else int(k)
    if k > ld:
        raise ValueError("k larger than the row length")
    wp = np.ascontiguousarray(wp, dtype=np.uint64)
    if wp.ndim != 2 or wp.shape[1] != words(k):
        raise ValueError(f"packed weights must be (rows, {words(k)}) for K={k}")
    x_bits = np.ascontiguousarray(x_bits)
    N = wp.shape[0]
    s = np.zeros((M, N), dtype=np.float64)
    if M and N:
        _load().oracle_dot_signw_bf16(_ptr(x_bits), ld, _ptr(wp), M, N, k, _ptr(s), nthreads)
    return s


def dot_pairs(xp: np.ndarray, wp: np.ndarray, k: int, mi, ni) -> np.ndarray:
    """int32 ``<x_{mi[i]}, w_{ni[i]}>`` for sampled (m, n) pairs."""
    xp, wp = _check_packed(xp, wp, k)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    if mi.shape != ni.shape or mi.ndim != 1:
        raise ValueError("mi and ni must be 1-D and of equal length")
    if mi.size and (mi.min() < 0 or mi.max() >= xp.shape[0] or ni.min() < 0
                    or ni.max() >= wp.shape[0]):
        raise IndexError("sample index out of range")
    out = np.zeros(mi.shape, dtype=np.int32)
    if mi.size:
        _load().oracle_dot_pairs(_ptr(xp), _ptr(wp), k, _ptr(mi), _ptr(ni), mi.size, _ptr(out))
    return out


def chain(x, weights, alpha_last, nthreads: int = 0):
    """Chained binary layers: pack the input once, then each hidden layer is
    sign -> repack and the last layer is alpha-scaled fp32.  ``x`` is float32
    (or uint16 bf16 bits) ``(M, K0)``; ``weights`` is a list of float32
    ``(N_i, K_i)`` with ``K_{i+1} = N_i``.  Returns (final fp32, [packed
    hidden activations]) built from the primitive oracle calls in order."""
    h = pack(x)
    k = np.asarray(x).shape[1]
    hidden = []
    for i, w in enumerate(weights):
        wp = pack(np.asarray(w, dtype=np.float32))
        if i + 1 < len(weights):
            h = sign_repack(h, wp, k, nthreads)
            hidden.append(h)
            k = w.shape[0]
        else:
            return gemm_scaled(h, wp, alpha_last, k, nthreads), hidden
    raise ValueError("chain needs at least one layer")
