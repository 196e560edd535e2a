"""GPU parity for bnn_gemm_signw_bf16: real-valued bf16 activations times
packed sign weights (binary_nn README, "Binary Regression" and "Triton Kernel
Benchmark": the eval-only packed-sign path), against the float64 oracle.

Bar (derived from the arithmetic; the pages fix no precision beyond "differs
from the dense product by rounding"):
  * exact regime -- integer-valued activations with |partial sums| < 2^24:
    every fp32 partial sum is exact in any order, so the kernel's output must
    equal fp32(s) * alpha[n] (one round-to-nearest-even product) bit for bit;
  * general inputs -- |y - alpha s| <= |alpha| gamma_K sum_k |x_k|
    + 2^-23 |y| + K 2^-126 |alpha|, gamma_K = K u / (1 - K u) with u = 2^-23:
    the standard bound for a K-term fp32 sum in any order (Higham, "Accuracy
    and Stability of Numerical Algorithms", eq. 4.4), with u doubled so that
    a unit that does not round to nearest (the MFMA accumulator, v_dot2) is
    covered, plus the alpha product and flushed subnormal products.
Each kernel family is forced through the algo selector and checked on its own.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import packed_xor_popcount_amd as bnn

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
U = 2.0 ** -23


def say(*a):
    print(*a, flush=True)


def to_dev_words(p: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(p, dtype=np.uint64).view(np.int64)).to(DEV)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rand_bf16(rng, rows, k):
    f = rng.standard_normal((rows, k)).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def int_bf16(rng, rows, k, lim=64):
    """Integer values in [-lim, lim] (exact in bf16), some exact zeros."""
    v = rng.integers(-lim, lim + 1, size=(rows, k)).astype(np.float32)
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rand_packed(rng, rows, k):
    kw = oracle.words(k)
    return rng.integers(0, 2 ** 64, size=(rows, kw), dtype=np.uint64)  # garbage pads included


def assert_exact(got, s, alpha):
    ref = s.astype(np.float32)
    assert np.array_equal(ref.astype(np.float64), s)  # the regime really is exact
    if alpha is not None:
        ref = ref * alpha[None, :].astype(np.float32)
    nz = ref != 0
    assert np.array_equal(got[nz].view(np.uint32), ref[nz].view(np.uint32))
    assert np.all(got[~nz] == 0)


def assert_within_bound(got, s, alpha, absx, K):
    a = np.ones(s.shape[1]) if alpha is None else np.abs(alpha.astype(np.float64))
    ref = s if alpha is None else s * alpha.astype(np.float64)[None, :]
    gamma = K * U / (1 - K * U)
    bound = a[None, :] * (gamma * absx[:, None] + K * 2.0 ** -126) + U * np.abs(got)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-300)).max())


SHAPES = [
    (1, 1, 1), (1, 256, 512), (1, 4096, 4096), (3, 100, 65), (8, 300, 1000), (2, 130, 4000),
    (9, 77, 129), (33, 257, 129), (64, 1000, 1000), (130, 513, 4095), (256, 1024, 1024),
    (5, 64, 0), (40, 70, 2049),
]


def algos_for(M, K):
    out = [bnn.ALGO_MFMA, bnn.ALGO_AUTO]
    if 1 <= M <= 8 and K > 0 and M * oracle.words(K) * 144 <= 65536:
        out.append(bnn.ALGO_GEMV)
    return out


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_signw_exact_regime(M, N, K):
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    xb = int_bf16(rng, M, K)
    wp = rand_packed(rng, N, K)
    alpha = (rng.standard_normal(N) * 2).astype(np.float32)
    alpha[::7] = 0.0
    s = oracle.dot_signw_bf16(xb, wp, K)
    xd, wd, ad = bf16_dev(xb), to_dev_words(wp), torch.from_numpy(alpha).to(DEV)
    for algo in algos_for(M, K):
        say("signw exact", M, N, K, "algo", algo)
        assert_exact(bnn.gemm_signw_bf16(xd, wd, K, None, algo).cpu().numpy(), s, None)
        assert_exact(bnn.gemm_signw_bf16(xd, wd, K, ad, algo).cpu().numpy(), s, alpha)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_signw_general_inputs(M, N, K):
    rng = np.random.default_rng(M * 17 + N * 3 + K + 5)
    xb = rand_bf16(rng, M, K)
    wp = rand_packed(rng, N, K)
    alpha = (np.abs(rng.standard_normal(N)) + 0.01).astype(np.float32)
    s = oracle.dot_signw_bf16(xb, wp, K)
    absx = np.abs(bf16_values(xb)).sum(axis=1)
    xd, wd, ad = bf16_dev(xb), to_dev_words(wp), torch.from_numpy(alpha).to(DEV)
    for algo in algos_for(M, K):
        say("signw general", M, N, K, "algo", algo)
        assert_within_bound(bnn.gemm_signw_bf16(xd, wd, K, ad, algo).cpu().numpy(), s, alpha,
                            absx, K)


def test_signw_strided_and_unaligned_rows():
    rng = np.random.default_rng(40)
    M, N, K = 37, 150, 700
    big = int_bf16(rng, M, K + 9)
    wp = rand_packed(rng, N, K)
    wd = to_dev_words(wp)
    dbig = bf16_dev(big)
    # row stride K + 9 (odd: 8-byte loads impossible), first K columns
    view = dbig[:, :K]
    s = oracle.dot_signw_bf16(np.ascontiguousarray(big[:, :K]), wp, K)
    for algo in (bnn.ALGO_MFMA, bnn.ALGO_AUTO):
        assert_exact(bnn.gemm_signw_bf16(view, wd, K, None, algo).cpu().numpy(), s, None)
    # a view starting one element in (2-byte aligned only), contiguous rows
    flat = bf16_dev(int_bf16(rng, 1, 1 + 4 * K).ravel())
    x4 = flat[1:].view(4, K)
    assert x4.data_ptr() % 8 != 0
    s4 = oracle.dot_signw_bf16(np.ascontiguousarray(
        x4.cpu().view(torch.int16).numpy().view(np.uint16)), wp, K)
    for algo in (bnn.ALGO_MFMA, bnn.ALGO_GEMV):
        assert_exact(bnn.gemm_signw_bf16(x4, wd, K, None, algo).cpu().numpy(), s4, None)


@pytest.mark.parametrize("M,K", [(1, 4096), (1, 20), (3, 1000), (8, 2049), (2, 96), (5, 4163)])
@pytest.mark.parametrize("off,pad", [(0, 0), (4, 0), (0, 4), (8, 8), (1, 0), (0, 9)])
def test_signw_gemv_staging_alignments(M, K, off, pad):
    """The batch GEMV stages the activation rows from 8-byte pieces (row
    starts 8-byte aligned) or element by element (else, and for pieces that
    reach past K): row starts at every alignment (offsets of 0, 1, 4 and 8
    elements, row strides K + 0/4/8/9), ragged last chunks and K below one
    chunk, against the oracle bit for bit."""
    rng = np.random.default_rng(M * 1000 + K + 17 * off + pad)
    N = 300
    ld = K + pad
    flat = int_bf16(rng, 1, off + M * ld + 16).ravel()
    dflat = bf16_dev(flat)
    view = dflat[off:off + M * ld].view(M, ld)[:, :K]
    xb = np.ascontiguousarray(flat[off:off + M * ld].reshape(M, ld)[:, :K])
    wp = rand_packed(rng, N, K)
    alpha = (rng.standard_normal(N) * 2).astype(np.float32)
    s = oracle.dot_signw_bf16(xb, wp, K)
    say("signw gemv staging", M, K, "offset", off, "pad", pad, "ptr % 16", view.data_ptr() % 16)
    got = bnn.gemm_signw_bf16(view, to_dev_words(wp), K, torch.from_numpy(alpha).to(DEV),
                              bnn.ALGO_GEMV)
    assert_exact(got.cpu().numpy(), s, alpha)


def test_signw_gemv_rejects_oversized_rows():
    x = torch.zeros(2, 70001, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(3, oracle.words(70001), dtype=torch.int64, device=DEV)
    with pytest.raises(bnn.BnnError):
        bnn.gemm_signw_bf16(x, w, 70001, None, bnn.ALGO_GEMV)
    y = bnn.gemm_signw_bf16(x, w, 70001)  # AUTO takes the matrix-core kernel
    assert y.shape == (2, 3) and not y.any()


@pytest.mark.parametrize("M,K,N", [(256, 1024, 1024), (512, 2048, 2048), (16384, 1024, 1024)])
def test_signw_page_shapes_every_output(M, K, N):
    # the packed-sign kernel shapes of the "Triton Kernel Benchmark" section,
    # N(0,1) activations and weights; every output against the oracle's
    # float64 sums (16384 x 1024 x 1024: a few seconds of host time)
    g = torch.Generator().manual_seed(M + K)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = torch.randn(N, K, generator=g)
    wd = bnn.pack_signs(w.to(DEV))
    wp = oracle.pack(w.numpy())
    assert np.array_equal(wd.cpu().numpy().view(np.uint64), wp)
    alpha = w.abs().mean(dim=1).numpy().astype(np.float32)
    y = bnn.gemm_signw_bf16(x.to(DEV), wd, K, torch.from_numpy(alpha).to(DEV)).cpu().numpy()
    xb = x.view(torch.int16).numpy().view(np.uint16)
    s = oracle.dot_signw_bf16(np.ascontiguousarray(xb), wp, K)
    absx = np.abs(bf16_values(xb)).sum(axis=1)
    assert_within_bound(y, s, alpha, absx, K)
