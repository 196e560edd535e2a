"""C-ABI checks that need no GPU: libbnn.so loads, exports every entry point
include/bnn.h declares, and rejects invalid arguments on the host before any
launch (so these calls never reach the device)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import packed_xor_popcount_amd as bnn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bnn.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_LAUNCH, E_ARG = range(7)
P = ctypes.c_void_p
FAKE = P(0x1000)        # aligned, never dereferenced: every call below fails validation
FAKE_ODD = P(0x1003)    # misaligned


def declared_symbols(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bnn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return bnn.library()


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for s in ("bnn_pack_signs", "bnn_gemm_u64", "bnn_gemm_u64_scaled", "bnn_gemm_sign_repack"):
        assert s in syms
    assert set(syms) == set(bnn.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bnn.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)", out))
    for s in declared_symbols():
        assert s in exported, s
        assert hasattr(lib, s)


def test_calibration_library_exports_its_header():
    """libbnn_calib.so (the benchmark's rate probes) loads and exports every
    entry point include/bnn_calib.h declares; libbnn.so does not need it."""
    from packed_xor_popcount_amd import calib
    header = os.path.join(ROOT, "include", "bnn_calib.h")
    syms = declared_symbols(header)
    assert set(syms) == set(calib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", calib.library_path],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)", out))
    lib = calib.library()
    for s in syms:
        assert s in exported, s
        assert hasattr(lib, s)
    # host-side validation, no launch
    assert lib.bnn_calib_valu(None, 1, 1, None) == E_NULL
    assert lib.bnn_calib_mfma_fp4(FAKE, 0, 1, None) == E_SHAPE
    assert lib.bnn_calib_mfma_fp4_pm1(FAKE, 1, 0, None) == E_SHAPE
    assert lib.bnn_calib_mfma_fp4_pm1(None, 1, 1, None) == E_NULL
    assert lib.bnn_calib_read(FAKE, 15, FAKE, 1, None) == E_SHAPE
    assert lib.bnn_calib_read(FAKE_ODD, 16, FAKE, 1, None) == E_ALIGN
    deps = subprocess.run(["readelf", "-d", bnn.library_path], capture_output=True, text=True,
                          check=True).stdout
    assert "bnn_calib" not in deps


def test_library_is_gfx950_code():
    # the offload target triple of the embedded device code object
    with open(bnn.library_path, "rb") as f:
        blob = f.read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_words_and_strings(lib):
    for k in (-5, 0, 1, 63, 64, 65, 1000, 4096, 2 ** 31):
        assert bnn.words(k) == (0 if k <= 0 else -(-k // 64))
    for s in range(7):
        assert lib.bnn_status_str(s)
    assert b"unknown" in lib.bnn_status_str(99)
    assert "gfx950" in bnn.version()


def test_pack_validation(lib):
    f = lib.bnn_pack_signs
    assert f(FAKE, 7, 1, 1, 1, FAKE, None) == E_DTYPE
    assert f(FAKE, 0, -1, 1, 1, FAKE, None) == E_SHAPE
    assert f(FAKE, 0, 1, -1, 1, FAKE, None) == E_SHAPE
    assert f(FAKE, 0, 2, 10, 9, FAKE, None) == E_SHAPE        # ld < k
    assert f(FAKE, 0, 2 ** 30, 1, 1, FAKE, None) == E_SHAPE    # too many rows
    assert f(None, 0, 2, 10, 10, FAKE, None) == E_NULL
    assert f(FAKE, 0, 2, 10, 10, None, None) == E_NULL
    assert f(FAKE_ODD, 0, 2, 10, 10, FAKE, None) == E_ALIGN   # fp32 needs 4 B
    assert f(P(0x1002), 1, 2, 10, 10, P(0x1004), None) == E_ALIGN  # dst needs 8 B
    # empty inputs: OK, nothing launched, NULL allowed
    assert f(None, 0, 0, 10, 10, None, None) == OK
    assert f(None, 1, 5, 0, 0, None, None) == OK


def test_gemm_validation(lib):
    g = lib.bnn_gemm_ex
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 3, 0, None) == E_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 0, 9, None) == E_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 1, 2 ** 24 + 1, 0, 3, None) == E_SHAPE  # MFMA K limit
    assert g(FAKE, FAKE, FAKE, FAKE, -1, 1, 1, 0, 0, None) == E_SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, 1, -1, 1, 0, 0, None) == E_SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 1, -1, 0, 0, None) == E_SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 1, 2 ** 30, 0, 0, None) == E_SHAPE
    assert g(None, FAKE, FAKE, FAKE, 1, 1, 1, 0, 0, None) == E_NULL
    assert g(FAKE, None, FAKE, FAKE, 1, 1, 1, 0, 0, None) == E_NULL
    assert g(FAKE, FAKE, FAKE, None, 1, 1, 1, 0, 0, None) == E_NULL
    assert g(FAKE, FAKE, None, FAKE, 1, 1, 1, 1, 0, None) == E_NULL   # scaled needs alpha
    assert g(FAKE_ODD, FAKE, FAKE, FAKE, 1, 1, 1, 0, 0, None) == E_ALIGN
    assert g(FAKE, FAKE_ODD, FAKE, FAKE, 1, 1, 1, 0, 0, None) == E_ALIGN
    assert g(FAKE, FAKE, FAKE, P(0x1002), 1, 1, 1, 0, 0, None) == E_ALIGN
    assert g(FAKE, FAKE, FAKE, P(0x1004), 1, 1, 1, 2, 0, None) == E_ALIGN  # repack words: 8 B
    assert g(FAKE, FAKE, P(0x1001), FAKE, 1, 1, 1, 1, 0, None) == E_ALIGN
    # the named entry points validate the same way
    assert lib.bnn_gemm_u64(None, FAKE, FAKE, 1, 1, 1, None) == E_NULL
    assert lib.bnn_gemm_u64_scaled(FAKE, FAKE, None, FAKE, 1, 1, 1, None) == E_NULL
    assert lib.bnn_gemm_sign_repack(FAKE, FAKE, FAKE_ODD, 1, 1, 1, None) == E_ALIGN
    # empty products: OK without a launch, NULLs allowed for empty buffers
    assert g(None, FAKE, None, None, 0, 5, 64, 0, 0, None) == OK
    assert g(FAKE, None, None, None, 5, 0, 64, 1, 0, None) == OK
    assert g(None, None, None, None, 0, 0, 64, 2, 0, None) == OK
    assert lib.bnn_gemm_u64(None, None, None, 0, 0, 0, None) == OK
    # a buffer with elements may not be NULL even when the product is empty
    assert g(None, None, None, None, 0, 5, 64, 0, 0, None) == E_NULL


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        bnn.pack_signs(torch.zeros(2, 3))
    with pytest.raises(TypeError):
        bnn.gemm_u64(torch.zeros(2, 1, dtype=torch.int64), torch.zeros(2, 1, dtype=torch.int64), 3)


def test_gemv_act_validation(lib):
    f = lib.bnn_gemv_act
    assert f(FAKE, 5, 4, FAKE, FAKE, FAKE, 1, 1, 4, 0, None) == E_DTYPE
    assert f(FAKE, 0, 4, FAKE, FAKE, FAKE, 1, 1, 4, 7, None) == E_ARG
    assert f(FAKE, 0, 3, FAKE, FAKE, FAKE, 1, 1, 4, 0, None) == E_SHAPE    # ldx < K
    assert f(FAKE, 0, 4, FAKE, FAKE, FAKE, -1, 1, 4, 0, None) == E_SHAPE
    assert f(None, 0, 4, FAKE, FAKE, FAKE, 1, 1, 4, 0, None) == E_NULL
    assert f(FAKE, 0, 4, None, FAKE, FAKE, 1, 1, 4, 0, None) == E_NULL
    assert f(FAKE, 0, 4, FAKE, None, FAKE, 1, 1, 4, 1, None) == E_NULL
    assert f(P(0x1002), 0, 4, FAKE, FAKE, FAKE, 1, 1, 4, 0, None) == E_ALIGN   # fp32 x
    assert f(P(0x1001), 1, 4, FAKE, FAKE, FAKE, 1, 1, 4, 0, None) == E_ALIGN   # bf16 x
    assert f(FAKE, 1, 4, FAKE_ODD, FAKE, FAKE, 1, 1, 4, 0, None) == E_ALIGN
    assert f(FAKE, 1, 4, FAKE, FAKE, P(0x1004), 1, 1, 4, 2, None) == E_ALIGN
    assert f(None, 0, 4, FAKE, None, None, 0, 3, 4, 0, None) == OK


def test_repack_thr_validation(lib):
    f = lib.bnn_gemm_sign_repack_thr
    # (xp, wp, thr, flip, yp, M, N, K, algo, stream)
    assert f(FAKE, FAKE, FAKE, None, FAKE, 1, 1, 64, 9, None) == E_ARG
    assert f(FAKE, FAKE, FAKE, None, FAKE, -1, 1, 64, 0, None) == E_SHAPE
    assert f(FAKE, FAKE, FAKE, None, FAKE, 1, 1, 2 ** 24 + 1, 3, None) == E_SHAPE  # MFMA limit
    assert f(FAKE, FAKE, None, None, FAKE, 1, 1, 64, 0, None) == E_NULL            # thr
    assert f(None, FAKE, FAKE, None, FAKE, 1, 1, 64, 0, None) == E_NULL
    assert f(FAKE, FAKE, FAKE, None, None, 1, 1, 64, 0, None) == E_NULL
    assert f(FAKE, FAKE, P(0x1002), None, FAKE, 1, 1, 64, 0, None) == E_ALIGN      # thr
    assert f(FAKE, FAKE, FAKE, P(0x1004), FAKE, 1, 1, 64, 0, None) == E_ALIGN      # flip
    assert f(FAKE, FAKE, FAKE, None, P(0x1004), 1, 1, 64, 0, None) == E_ALIGN      # yp
    assert f(None, FAKE, None, None, None, 0, 3, 64, 0, None) == OK                # empty
    # the threshold epilogue is reachable only through its own entry point
    assert lib.bnn_gemm_ex(FAKE, FAKE, None, FAKE, 1, 1, 64, 3, 0, None) == E_ARG
    assert lib.bnn_gemv_act(FAKE, 0, 64, FAKE, None, FAKE, 1, 1, 64, 3, None) == E_ARG


def test_signw_validation(lib):
    f = lib.bnn_gemm_signw_bf16
    # (x, ldx, wp, alpha, y, M, N, K, algo, stream)
    assert f(FAKE, 64, FAKE, None, FAKE, 1, 1, 64, bnn.ALGO_TILED, None) == E_ARG
    assert f(FAKE, 64, FAKE, None, FAKE, 1, 1, 64, 9, None) == E_ARG
    assert f(FAKE, 63, FAKE, None, FAKE, 1, 1, 64, 0, None) == E_SHAPE      # ldx < K
    assert f(FAKE, 64, FAKE, None, FAKE, -1, 1, 64, 0, None) == E_SHAPE
    assert f(FAKE, 64, FAKE, None, FAKE, 9, 1, 64, bnn.ALGO_GEMV, None) == E_SHAPE  # M > 8
    assert f(FAKE, 2 ** 20, FAKE, None, FAKE, 1, 1, 2 ** 20, bnn.ALGO_GEMV, None) == E_SHAPE
    assert f(None, 64, FAKE, None, FAKE, 1, 1, 64, 0, None) == E_NULL
    assert f(FAKE, 64, None, None, FAKE, 1, 1, 64, 0, None) == E_NULL
    assert f(FAKE, 64, FAKE, None, None, 1, 1, 64, 0, None) == E_NULL
    assert f(P(0x1001), 64, FAKE, None, FAKE, 1, 1, 64, 0, None) == E_ALIGN  # bf16 x
    assert f(FAKE, 64, FAKE_ODD, None, FAKE, 1, 1, 64, 0, None) == E_ALIGN
    assert f(FAKE, 64, FAKE, P(0x1002), FAKE, 1, 1, 64, 0, None) == E_ALIGN  # alpha
    assert f(FAKE, 64, FAKE, None, P(0x1002), 1, 1, 64, 0, None) == E_ALIGN  # y
    assert f(None, 64, FAKE, None, None, 0, 3, 64, 0, None) == OK            # empty


def test_chain3_validation(lib):
    # (x, dtype, ldx, w1, thr1, flip1, w2, thr2, flip2, w3, alpha3, y, M, K0, N1, N2, N3, stream)
    def f(x, dt, ldx, w1, w2, w3, a3, y, M, *dims_stream, thr1=None, flip1=None):
        return lib.bnn_chain3(x, dt, ldx, w1, thr1, flip1, w2, None, None, w3, a3, y, M,
                              *dims_stream)
    ok_dims = (512, 256, 128, 64)
    assert f(FAKE, 7, 512, FAKE, FAKE, FAKE, None, FAKE, 4, *ok_dims, None) == E_DTYPE
    for dims in [(500, 256, 128, 64), (640, 256, 128, 64), (512, 192, 128, 64),
                 (512, 256, 64, 64), (512, 256, 128, 48), (512, 256, 128, 544),
                 (512, 512, 512, 512)]:   # the last: weights too large for LDS
        assert f(FAKE, 0, 1024, FAKE, FAKE, FAKE, None, FAKE, 4, *dims, None) == E_SHAPE, dims
    assert f(FAKE, 0, 511, FAKE, FAKE, FAKE, None, FAKE, 4, *ok_dims, None) == E_SHAPE  # ldx < K0
    assert f(FAKE, 0, 512, FAKE, FAKE, FAKE, None, FAKE, -1, *ok_dims, None) == E_SHAPE
    assert f(None, 0, 512, FAKE, FAKE, FAKE, None, FAKE, 4, *ok_dims, None) == E_NULL
    assert f(FAKE, 0, 512, FAKE, None, FAKE, None, FAKE, 4, *ok_dims, None) == E_NULL
    assert f(FAKE, 0, 512, FAKE, FAKE, FAKE, None, None, 4, *ok_dims, None) == E_NULL
    assert f(P(0x1002), 0, 512, FAKE, FAKE, FAKE, None, FAKE, 4, *ok_dims, None) == E_ALIGN
    assert f(FAKE, 0, 512, FAKE, FAKE, FAKE_ODD, None, FAKE, 4, *ok_dims, None) == E_ALIGN
    assert f(FAKE, 0, 512, FAKE, FAKE, FAKE, P(0x1001), FAKE, 4, *ok_dims, None) == E_ALIGN
    assert f(None, 1, 512, FAKE, FAKE, FAKE, None, None, 0, *ok_dims, None) == OK     # M = 0
    assert f(FAKE, 0, 512, FAKE, FAKE, FAKE, None, FAKE, 4, *ok_dims, None,
             thr1=P(0x1002)) == E_ALIGN
    assert f(FAKE, 0, 512, FAKE, FAKE, FAKE, None, FAKE, 4, *ok_dims, None,
             flip1=P(0x1004)) == E_ALIGN
