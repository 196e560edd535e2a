"""Seeded random-shape parity sweep on the GPU: every kernel family and
epilogue of the packed products, the threshold repack, the real-activation
product on both kernels, and the fused chain, each at random ragged sizes
against the CPU oracle (same bars as the other parity tests: packed words and
int32 bit-exact, scaled fp32 bit-identical, real-activation sums exact in the
integer regime).  Shapes are drawn once per seed, so a failure names its case."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import packed_xor_popcount_amd as bnn
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ALGOS = [bnn.ALGO_GEMV, bnn.ALGO_TILED, bnn.ALGO_MFMA, bnn.ALGO_AUTO]


def dev_words(p):
    return torch.from_numpy(np.ascontiguousarray(p, np.uint64).view(np.int64)).to(DEV)


def host_words(t):
    return t.cpu().numpy().view(np.uint64)


def scaled_equal(got, ref):
    nz = ref != 0
    return np.array_equal(got[nz].view(np.uint32), ref[nz].view(np.uint32)) and not got[~nz].any()


def shape(seed):
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.choice([1, 2, 5, 8, 9, 33, int(rng.integers(1, 200))]))
    N = int(rng.integers(1, 700))
    K = int(rng.choice([0, 1, 63, 64, 65, int(rng.integers(1, 2500))]))
    return rng, M, N, K


@pytest.mark.parametrize("seed", range(24))
def test_random_products(seed):
    rng, M, N, K = shape(seed)
    print("random products", seed, M, N, K, flush=True)
    kw = oracle.words(K)
    xg = rng.integers(0, 2 ** 64, size=(M, kw), dtype=np.uint64)  # garbage pad bits
    wg = rng.integers(0, 2 ** 64, size=(N, kw), dtype=np.uint64)
    xc, wc = xg.copy(), wg.copy()
    if kw and K % 64:
        keep = np.uint64((1 << (K % 64)) - 1)
        xc[:, -1] &= keep
        wc[:, -1] &= keep
    alpha = (rng.standard_normal(N) * 2).astype(np.float32)
    thr = rng.integers(-K - 2, K + 3, N).astype(np.int32)
    mask = rng.integers(0, 2 ** 64, size=oracle.words(N), dtype=np.uint64)
    flags = np.unpackbits(mask.view(np.uint8), bitorder="little")[:N].astype(np.uint8)
    ref_i = oracle.gemm_i32(xc, wc, K)
    ref_s = oracle.gemm_scaled(xc, wc, alpha, K)
    ref_p = oracle.sign_repack(xc, wc, K)
    ref_t = oracle.sign_repack_thr(xc, wc, thr, K, flags)
    xd, wd, ad = dev_words(xg), dev_words(wg), torch.from_numpy(alpha).to(DEV)
    td, fd = torch.from_numpy(thr).to(DEV), dev_words(mask)
    for algo in ALGOS:
        assert np.array_equal(bnn.gemm_ex(xd, wd, K, bnn.EPI_I32, algo).cpu().numpy(), ref_i), algo
        assert scaled_equal(bnn.gemm_ex(xd, wd, K, bnn.EPI_SCALED, algo, alpha=ad).cpu().numpy(),
                            ref_s), algo
        assert np.array_equal(host_words(bnn.gemm_ex(xd, wd, K, bnn.EPI_REPACK, algo)), ref_p), algo
        assert np.array_equal(host_words(bnn.gemm_sign_repack_thr(xd, wd, td, K, fd, algo)),
                              ref_t), algo


@pytest.mark.parametrize("seed", range(12))
def test_random_real_activation_products(seed):
    rng, M, N, K = shape(seed + 100)
    K = max(K, 1)
    print("random signw", seed, M, N, K, flush=True)
    v = rng.integers(-32, 33, size=(M, K)).astype(np.float32)  # exact partial sums
    xb = (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    wp = rng.integers(0, 2 ** 64, size=(N, oracle.words(K)), dtype=np.uint64)
    alpha = (np.abs(rng.standard_normal(N)) + 0.1).astype(np.float32)
    s = oracle.dot_signw_bf16(xb, wp, K)
    ref = s.astype(np.float32) * alpha[None, :]
    xd = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV)
    algos = [bnn.ALGO_MFMA, bnn.ALGO_AUTO]
    if M <= 8 and M * oracle.words(K) * 144 <= 65536:
        algos.append(bnn.ALGO_GEMV)
    for algo in algos:
        got = bnn.gemm_signw_bf16(xd, dev_words(wp), K, torch.from_numpy(alpha).to(DEV), algo)
        assert scaled_equal(got.cpu().numpy(), ref), algo


@pytest.mark.parametrize("seed", range(8))
def test_random_fused_chains(seed):
    rng = np.random.default_rng(2000 + seed)
    dims = [int(rng.choice([128, 256, 384, 512])) for _ in range(3)] + \
           [int(32 * rng.integers(1, 9))]
    M = int(rng.integers(1, 400))
    kw = [d // 64 for d in dims[:3]]
    if (dims[1] * kw[0] + dims[2] * kw[1] + dims[3] * kw[2] + (dims[1] + dims[2]) // 2
            + kw[1] + kw[2] + 128 * sum(kw)) * 8 > 64 * 1024:
        dims = [256, 256, 128, 64]
    print("random chain", seed, M, dims, flush=True)
    g = workloads.generator(3000 + seed)
    dt = torch.bfloat16 if seed % 2 else torch.float32
    x = workloads.normal(g, M, dims[0]).to(dt)
    ws = [workloads.normal(g, dims[i + 1], dims[i]).numpy() for i in range(3)]
    alpha = workloads.absmean_alpha(torch.from_numpy(ws[2])).numpy()
    thr = [rng.integers(-dims[i] - 2, dims[i] + 3, dims[i + 1]).astype(np.int32) for i in range(2)]
    masks = [rng.integers(0, 2 ** 64, size=oracle.words(dims[i + 1]), dtype=np.uint64)
             for i in range(2)]
    flags = [np.unpackbits(m.view(np.uint8), bitorder="little")[:dims[i + 1]].astype(np.uint8)
             for i, m in enumerate(masks)]
    xh = workloads.bf16_bits(x) if dt == torch.bfloat16 else x.numpy()
    h = oracle.pack(xh)
    k = dims[0]
    for i in range(2):
        h = oracle.sign_repack_thr(h, oracle.pack(ws[i]), thr[i], k, flags[i])
        k = dims[i + 1]
    ref = oracle.gemm_scaled(h, oracle.pack(ws[2]), alpha, k)
    wd = [bnn.pack_signs(torch.from_numpy(w).to(DEV)) for w in ws]
    got = bnn.chain3(x.to(DEV), *wd, torch.from_numpy(alpha).to(DEV),
                     thr1=torch.from_numpy(thr[0]).to(DEV), flip1=dev_words(masks[0]),
                     thr2=torch.from_numpy(thr[1]).to(DEV), flip2=dev_words(masks[1]))
    assert scaled_equal(got.cpu().numpy(), ref)
