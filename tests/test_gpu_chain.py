"""GPU parity for bnn_chain3, the fused three-layer binary chain (pack ->
sign/repack -> sign/repack -> fp32), against the oracle's chain of primitive
calls ("Encoder / decoder", BinaryAutoEncoder; "Binary Math Effectiveness",
section 1 for every step).  Bar: bit-exact -- the hidden layers are packed
words and the last layer is the same one-multiply alpha product of an exact
integer as bnn_gemm_u64_scaled."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import packed_xor_popcount_amd as bnn
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def words_np(t):
    return t.cpu().numpy().view(np.uint64)


def assert_scaled_equal(got, ref):
    nz = ref != 0
    assert np.array_equal(got[nz].view(np.uint32), ref[nz].view(np.uint32))
    assert np.all(got[~nz] == 0)


def oracle_chain(x_host, ws, alpha):
    """pack -> sign_repack -> sign_repack -> scaled (or int32 as fp32)."""
    h = oracle.pack(x_host)
    k = x_host.shape[1]
    for w in ws[:2]:
        h = oracle.sign_repack(h, oracle.pack(w), k)
        k = w.shape[0]
    w3 = oracle.pack(ws[2])
    if alpha is None:
        return oracle.gemm_i32(h, w3, k).astype(np.float32)
    return oracle.gemm_scaled(h, w3, alpha, k)


CASES = [
    (1, (512, 256, 128, 64)), (127, (512, 256, 128, 64)), (300, (128, 128, 128, 32)),
    (1000, (384, 256, 256, 96)), (129, (256, 384, 256, 128)), (64, (512, 384, 128, 256)),
    (33, (128, 512, 128, 512)),
]


@pytest.mark.parametrize("M,dims", CASES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chain3_parity(M, dims, dtype):
    say("chain3", M, dims, dtype)
    c = workloads.random_case(seed=M + sum(dims), M=M, N=1, K=dims[0], dist="normal",
                              zero_frac=0.01, dtype=dtype)
    x = c["x"]
    g = workloads.generator(7 * M + dims[1])
    ws = [workloads.normal(g, dims[i + 1], dims[i]).numpy() for i in range(3)]
    alpha = workloads.absmean_alpha(torch.from_numpy(ws[2])).numpy()
    alpha[::5] = 0.0
    xh = workloads.bf16_bits(x) if dtype == torch.bfloat16 else x.numpy()
    wd = [bnn.pack_signs(torch.from_numpy(w).to(DEV)) for w in ws]
    xd = x.to(DEV)
    got = bnn.chain3(xd, *wd, torch.from_numpy(alpha).to(DEV)).cpu().numpy()
    assert_scaled_equal(got, oracle_chain(xh, ws, alpha))
    got = bnn.chain3(xd, *wd, None).cpu().numpy()
    assert np.array_equal(got, oracle_chain(xh, ws, None))


def test_chain3_strided_rows():
    g = workloads.generator(90)
    big = workloads.normal(g, 70, 520)
    ws = [workloads.normal(g, 256, 512).numpy(), workloads.normal(g, 128, 256).numpy(),
          workloads.normal(g, 64, 128).numpy()]
    wd = [bnn.pack_signs(torch.from_numpy(w).to(DEV)) for w in ws]
    view = big.to(DEV)[:, 3:515]           # row stride 520, not 16-byte aligned rows
    got = bnn.chain3(view, *wd).cpu().numpy()
    assert np.array_equal(got, oracle_chain(np.ascontiguousarray(big.numpy()[:, 3:515]), ws, None))


@pytest.mark.parametrize("dims", [(500, 256, 128, 64), (512, 512, 512, 512)])
def test_chain3_rejects_unsupported_dims(dims):
    # K not a multiple of 128, or weights too large for the kernel's LDS
    x = torch.zeros(4, dims[0], device=DEV)
    w = [torch.zeros(dims[i + 1], bnn.words(dims[i]), dtype=torch.int64, device=DEV)
         for i in range(3)]
    with pytest.raises(bnn.BnnError):
        bnn.chain3(x, *w)


def test_chain3_workload_chain_65536():
    # the fused launch against the oracle and against the four separate
    # calls (the benchmark's unfused step), on every row
    d = workloads.make("chain_65536")
    dims = d["dims"]
    x = d["x"]
    xd = x.to(DEV)
    wd = [bnn.pack_signs(w.to(DEV)) for w in d["weights"]]
    ad = d["alpha"].to(DEV)
    y = bnn.chain3(xd, *wd, ad)
    h = bnn.pack_signs(xd)
    h1 = bnn.gemm_sign_repack(h, wd[0], dims[0])
    h2 = bnn.gemm_sign_repack(h1, wd[1], dims[1])
    y_sep = bnn.gemm_u64_scaled(h2, wd[2], ad, dims[2])
    assert torch.equal(y.view(torch.int32), y_sep.view(torch.int32))
    final, _ = oracle.chain(x.numpy(), [w.numpy() for w in d["weights"]], d["alpha"].numpy())
    assert_scaled_equal(y.cpu().numpy(), final)


# ---------------------------------------------------------------------------
# hidden layers as threshold repacks (a BatchNorm after each binary layer,
# folded: "Architecture Decision Record", Decision)


def _flags(mask, n):
    bits = np.unpackbits(np.ascontiguousarray(mask, np.uint64).view(np.uint8), bitorder="little")
    return bits[:n].astype(np.uint8)


def _rand_thr(rng, n, k):
    t = rng.integers(-k - 3, k + 3, n).astype(np.int64)
    t[:6] = [-(2 ** 31), 2 ** 31 - 1, -k - 1, -k, k, k - 1]
    return t.astype(np.int32)


def oracle_chain_thr(x_host, ws, alpha, thr, flags):
    h = oracle.pack(x_host)
    k = x_host.shape[1]
    for i, w in enumerate(ws[:2]):
        wp = oracle.pack(w)
        h = (oracle.sign_repack(h, wp, k) if thr[i] is None and flags[i] is None else
             oracle.sign_repack_thr(h, wp, thr[i] if thr[i] is not None
                                    else np.zeros(w.shape[0], np.int32), k, flags[i]))
        k = w.shape[0]
    return oracle.gemm_scaled(h, oracle.pack(ws[2]), alpha, k)


@pytest.mark.parametrize("M,dims", [(300, (512, 256, 128, 64)), (129, (256, 384, 256, 128)),
                                    (64, (512, 384, 128, 256))])
@pytest.mark.parametrize("which", ["both", "thr_only", "flip_only"])
def test_chain3_threshold_parity(M, dims, which):
    say("chain3 thr", M, dims, which)
    rng = np.random.default_rng(M + dims[1] + len(which))
    g = workloads.generator(11 * M + dims[2])
    x = workloads.normal(g, M, dims[0])
    ws = [workloads.normal(g, dims[i + 1], dims[i]).numpy() for i in range(3)]
    alpha = workloads.absmean_alpha(torch.from_numpy(ws[2])).numpy()
    thr = [_rand_thr(rng, dims[1], dims[0]), _rand_thr(rng, dims[2], dims[1])]
    masks = [rng.integers(0, 2 ** 64, size=bnn.words(dims[i + 1]), dtype=np.uint64)
             for i in range(2)]
    if which == "thr_only":
        masks = [None, None]
    if which == "flip_only":
        thr = [None, None]
    wd = [bnn.pack_signs(torch.from_numpy(w).to(DEV)) for w in ws]
    td = [None if t is None else torch.from_numpy(t).to(DEV) for t in thr]
    fd = [None if m is None else torch.from_numpy(m.view(np.int64)).to(DEV) for m in masks]
    got = bnn.chain3(x.to(DEV), *wd, torch.from_numpy(alpha).to(DEV), thr1=td[0], flip1=fd[0],
                     thr2=td[1], flip2=fd[1]).cpu().numpy()
    flags = [None if m is None else _flags(m, dims[i + 1]) for i, m in enumerate(masks)]
    assert_scaled_equal(got, oracle_chain_thr(x.numpy(), ws, alpha, thr, flags))


def test_chain3_workload_chain_65536_bn_folded():
    from packed_xor_popcount_amd.fold import bn_fold
    d = workloads.make("chain_65536")
    dims = d["dims"]
    x = d["x"]
    rng = np.random.default_rng(58)
    thr, flips = [], []
    for i in range(2):
        n, k = dims[i + 1], dims[i]
        t, f = bn_fold(rng.standard_normal(n), rng.standard_normal(n),
                       rng.standard_normal(n) * np.sqrt(k), np.abs(rng.standard_normal(n)) + 0.5,
                       np.ones(n), k)
        thr.append(t)
        flips.append(f)
    xd = x.to(DEV)
    wd = [bnn.pack_signs(w.to(DEV)) for w in d["weights"]]
    ad = d["alpha"].to(DEV)
    td = [torch.from_numpy(t).to(DEV) for t in thr]
    fd = [bnn.flip_words(torch.from_numpy(f).to(DEV)) for f in flips]
    y = bnn.chain3(xd, *wd, ad, thr1=td[0], flip1=fd[0], thr2=td[1], flip2=fd[1])
    h = bnn.pack_signs(xd)
    h1 = bnn.gemm_sign_repack_thr(h, wd[0], td[0], dims[0], fd[0])
    h2 = bnn.gemm_sign_repack_thr(h1, wd[1], td[1], dims[1], fd[1])
    y_sep = bnn.gemm_u64_scaled(h2, wd[2], ad, dims[2])
    assert torch.equal(y.view(torch.int32), y_sep.view(torch.int32))
    ref = oracle_chain_thr(x.numpy(), [w.numpy() for w in d["weights"]], d["alpha"].numpy(),
                           thr, flips)
    assert_scaled_equal(y.cpu().numpy(), ref)  # every row
