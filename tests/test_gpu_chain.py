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
    # the fused launch against the oracle on sampled rows, and against the
    # four separate calls (the benchmark's unfused step) on every row
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
    rng = np.random.default_rng(57)
    rows = np.sort(rng.choice(x.shape[0], 2048, replace=False))
    rows[0], rows[-1] = 0, x.shape[0] - 1
    final, _ = oracle.chain(x.numpy()[rows], [w.numpy() for w in d["weights"]], d["alpha"].numpy())
    assert_scaled_equal(y.cpu().numpy()[rows], final)
