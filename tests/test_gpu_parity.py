"""GPU parity: every HIP kernel behind include/bnn.h against the CPU oracle,
element by element, on the same seeded inputs.

Bar: packed words and int32 outputs bit-exact; alpha-scaled fp32 within
1e-6 relative (the bar the workload statement sets) -- and in fact
bit-identical, since both sides take one round-to-nearest-even fp32 product
of the same exactly converted integer; zeros compare by value (+0 == -0).

Sizes span several tiles and ragged tails (tile = 32 rows x 256 columns x
8 words for the tiled kernel; 64 columns per step for the GEMV kernel);
every kernel family is forced explicitly through bnn_gemm_ex, and the named
entry points are checked with their automatic choice.  The full-size
workloads are checked in the launch configuration the benchmark times, on
outputs the oracle computes one by one.
"""
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


def say(*a):
    print(*a, flush=True)


def to_dev_words(p: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(p, dtype=np.uint64).view(np.int64)).to(DEV)


def words_np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


def host_input(x: torch.Tensor) -> np.ndarray:
    """The exact bytes the oracle packs: fp32 values or bf16 bit patterns."""
    return workloads.bf16_bits(x) if x.dtype == torch.bfloat16 else x.numpy()


def assert_scaled_equal(got: np.ndarray, ref: np.ndarray):
    assert got.shape == ref.shape and got.dtype == np.float32
    nz = ref != 0
    rel = np.abs(got[nz].astype(np.float64) - ref[nz]) / np.abs(ref[nz].astype(np.float64))
    assert rel.size == 0 or rel.max() <= 1e-6
    assert np.array_equal(got[nz].view(np.uint32), ref[nz].view(np.uint32))
    assert np.all(got[~nz] == 0)


def rand_packed(rng, rows, k, garbage=True):
    """Random packed rows; optionally with garbage in the pad bits, which
    every product must ignore."""
    kw = oracle.words(k)
    p = rng.integers(0, 2 ** 64, size=(rows, kw), dtype=np.uint64)
    if kw and k % 64:
        keep = np.uint64((1 << (k % 64)) - 1)
        clean = p.copy()
        clean[:, -1] &= keep
        return (p if garbage else clean), clean
    return p, p


# ---------------------------------------------------------------------------
# bnn_pack_signs


@pytest.mark.parametrize("rows,k", [(1, 1), (1, 63), (3, 64), (5, 65), (7, 1000), (64, 4096),
                                    (130, 333), (1000, 129), (2, 5000), (4097, 40)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pack_parity(rows, k, dtype):
    say("pack", rows, k, dtype)
    g = workloads.generator(rows * 7919 + k)
    x = workloads.plant_zeros(g, workloads.normal(g, rows, k), 0.02) if rows * k >= 2 else \
        workloads.normal(g, rows, k)
    x = x.to(dtype)
    got = words_np(bnn.pack_signs(x.to(DEV)))
    ref = oracle.pack(host_input(x))
    assert np.array_equal(got, ref)


def test_pack_projection_tables():
    from tests import _golden
    f32 = np.array([b for b, _, _ in _golden.projection_f32()], dtype=np.uint32)
    exp = np.array([bit for _, _, bit in _golden.projection_f32()], dtype=np.uint64)
    x = torch.from_numpy(f32.view(np.float32).reshape(1, -1).copy())
    got = words_np(bnn.pack_signs(x.to(DEV)))[0, 0]
    assert got == np.sum(exp << np.arange(exp.size, dtype=np.uint64))
    b16 = np.array([b for b, _, _ in _golden.projection_bf16()], dtype=np.uint16)
    exp = np.array([bit for _, _, bit in _golden.projection_bf16()], dtype=np.uint64)
    x = torch.from_numpy(b16.view(np.int16).reshape(1, -1).copy()).view(torch.bfloat16)
    got = words_np(bnn.pack_signs(x.to(DEV)))[0, 0]
    assert got == np.sum(exp << np.arange(exp.size, dtype=np.uint64))


def test_pack_strided_rows_and_prefix():
    g = workloads.generator(77)
    big = workloads.normal(g, 33, 300).to(DEV)
    view = big[:, 10:210]                       # row stride 300, 200 columns
    got = words_np(bnn.pack_signs(view, k=150))  # first 150 of them
    ref = oracle.pack(np.ascontiguousarray(big.cpu().numpy()[:, 10:160]))
    assert np.array_equal(got, ref)


def test_pack_empty():
    assert bnn.pack_signs(torch.empty(0, 10, device=DEV)).shape == (0, 1)
    assert bnn.pack_signs(torch.empty(4, 0, device=DEV)).shape == (4, 0)


# ---------------------------------------------------------------------------
# products, every kernel family, ragged shapes, garbage pad bits

SHAPES = [
    (1, 1, 1), (1, 5, 0), (3, 64, 64), (1, 256, 512), (2, 300, 65), (8, 1000, 1000),
    (9, 65, 127), (33, 257, 129), (64, 1000, 1000), (65, 513, 4095), (100, 64, 8192),
    (31, 255, 63), (256, 256, 512), (5, 1025, 3000), (40, 130, 2049),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("algo", ALGOS)
def test_gemm_all_epilogues(M, N, K, algo):
    say("gemm", M, N, K, "algo", algo)
    rng = np.random.default_rng(M * 1000003 + N * 1009 + K)
    xg, xc = rand_packed(rng, M, K)
    wg, wc = rand_packed(rng, N, K)
    alpha = (rng.standard_normal(N) * 3).astype(np.float32)
    alpha[::5] = 0.0
    xd, wd, ad = to_dev_words(xg), to_dev_words(wg), torch.from_numpy(alpha).to(DEV)

    ref = oracle.gemm_i32(xc, wc, K)
    got = bnn.gemm_ex(xd, wd, K, bnn.EPI_I32, algo).cpu().numpy()
    assert np.array_equal(got, ref)

    refs = oracle.gemm_scaled(xc, wc, alpha, K)
    gots = bnn.gemm_ex(xd, wd, K, bnn.EPI_SCALED, algo, alpha=ad).cpu().numpy()
    assert_scaled_equal(gots, refs)

    refp = oracle.sign_repack(xc, wc, K)
    gotp = words_np(bnn.gemm_ex(xd, wd, K, bnn.EPI_REPACK, algo))
    assert np.array_equal(gotp, refp)


@pytest.mark.parametrize("K", [1000, 2049, 2304, 4163])
def test_mfma_large_tiles_ragged(K):
    # Large products with K >= 2048 run 320 x 192 block tiles of 5 x 3 wave
    # tiles (word outputs; 286 tiles in two rounds here) or 256 x 256 of
    # 4 x 4 (repacked outputs) on the matrix cores (K = 2049: a partial last
    # step; 2304: an odd number of whole steps; 4163: both), shorter K the
    # 256 x 64 tiles:
    # ragged M, N and K past every tile edge, garbage pad bits; the ragged
    # block row and block column are compared in full, the rest on sampled
    # outputs, for every epilogue.
    M, N = 16 * 256 + 37, 16 * 256 + 45
    say("mfma large tiles", M, N, K)
    rng = np.random.default_rng(K + 17)
    xg, xc = rand_packed(rng, M, K)
    wg, wc = rand_packed(rng, N, K)
    alpha = (rng.standard_normal(N) * 3).astype(np.float32)
    alpha[::5] = 0.0
    xd, wd, ad = to_dev_words(xg), to_dev_words(wg), torch.from_numpy(alpha).to(DEV)
    yi = bnn.gemm_ex(xd, wd, K, bnn.EPI_I32, bnn.ALGO_MFMA).cpu().numpy()
    ys = bnn.gemm_ex(xd, wd, K, bnn.EPI_SCALED, bnn.ALGO_MFMA, alpha=ad).cpu().numpy()
    yp = words_np(bnn.gemm_ex(xd, wd, K, bnn.EPI_REPACK, bnn.ALGO_MFMA))
    thr = rand_thr(rng, N, K)
    mask = rng.integers(0, 2 ** 64, size=oracle.words(N), dtype=np.uint64)
    yt = words_np(bnn.gemm_sign_repack_thr(xd, wd, torch.from_numpy(thr).to(DEV), K,
                                           to_dev_words(mask[None])[0], bnn.ALGO_MFMA))
    edge_r = np.arange(4096, M)
    edge_c = np.arange(4096, N)
    some_r = np.sort(rng.choice(4096, 40, replace=False))
    rows = np.concatenate([some_r, edge_r])
    ref_rows = oracle.gemm_i32(xc[rows], wc, K)
    assert np.array_equal(yi[rows], ref_rows)
    assert_scaled_equal(ys[rows], oracle.gemm_scaled(xc[rows], wc, alpha, K))
    assert np.array_equal(yp[rows], oracle.sign_repack(xc[rows], wc, K))
    assert np.array_equal(yt[rows], oracle.sign_repack_thr(xc[rows], wc, thr, K,
                                                           flags_of(mask, N)))
    ref_cols = oracle.gemm_i32(xc, wc[edge_c], K)
    assert np.array_equal(yi[:, edge_c], ref_cols)
    assert_scaled_equal(ys[:, edge_c], oracle.gemm_scaled(xc, wc[edge_c], alpha[edge_c], K))
    mi, ni = _sample_pairs(rng, M, N, 20000)
    assert np.array_equal(yi[mi, ni], oracle.dot_pairs(xc, wc, K, mi, ni))


@pytest.mark.parametrize("M,N,K", [(4389, 4392, 2049), (4389, 4392, 4096), (4389, 4392, 4163),
                                   (4389, 4392, 6000), (4389, 4392, 32767),
                                   (4000, 4072, 2049), (4000, 4072, 4163)])
def test_mfma_large_products_n_multiple_of_8(M, N, K):
    # Large products with N % 8 == 0: K = 4096 whole steps, 2049 and 4163 a
    # partial last step, 6000 an odd number of whole steps and a partial one,
    # 32767 a long K loop.  4389 x 4392 runs the word outputs on 320 x 192
    # block tiles (5 x 3 wave tiles: 322 tiles in two rounds against 324 of
    # 256 x 256), 4000 x 4072 on 256 x 256 (256 tiles, one round); the
    # repacked outputs always on 256 x 256.  Ragged block row and column
    # compared in full against the oracle, sampled outputs elsewhere, and
    # the whole product against the VALU kernel.
    say("mfma large products", M, N, K)
    rng = np.random.default_rng(K + 29)
    xg, xc = rand_packed(rng, M, K)
    wg, wc = rand_packed(rng, N, K)
    alpha = (rng.standard_normal(N) * 3).astype(np.float32)
    alpha[::7] = 0.0
    xd, wd, ad = to_dev_words(xg), to_dev_words(wg), torch.from_numpy(alpha).to(DEV)
    yi = bnn.gemm_ex(xd, wd, K, bnn.EPI_I32, bnn.ALGO_MFMA)
    ys = bnn.gemm_ex(xd, wd, K, bnn.EPI_SCALED, bnn.ALGO_MFMA, alpha=ad)
    assert torch.equal(yi, bnn.gemm_ex(xd, wd, K, bnn.EPI_I32, bnn.ALGO_TILED))
    assert torch.equal(ys, bnn.gemm_ex(xd, wd, K, bnn.EPI_SCALED, bnn.ALGO_TILED, alpha=ad))
    yi, ys = yi.cpu().numpy(), ys.cpu().numpy()
    # the last 320-row and 192-column block tiles (they contain the last
    # 256-row and 256-column ones' ragged edges too)
    edge_r = np.arange(min((M - 1) // 320 * 320, (M - 1) // 256 * 256), M)
    edge_c = np.arange(min((N - 1) // 192 * 192, (N - 1) // 256 * 256), N)
    assert np.array_equal(yi[edge_r], oracle.gemm_i32(xc[edge_r], wc, K))
    assert_scaled_equal(ys[edge_r], oracle.gemm_scaled(xc[edge_r], wc, alpha, K))
    assert np.array_equal(yi[:, edge_c], oracle.gemm_i32(xc, wc[edge_c], K))
    assert_scaled_equal(ys[:, edge_c], oracle.gemm_scaled(xc, wc[edge_c], alpha[edge_c], K))
    mi, ni = _sample_pairs(rng, M, N, 20000)
    d = oracle.dot_pairs(xc, wc, K, mi, ni)
    assert np.array_equal(yi[mi, ni], d)
    assert np.array_equal(ys[mi, ni], (d.astype(np.float32) * alpha[ni]).astype(np.float32))


def test_named_entry_points_match_oracle():
    rng = np.random.default_rng(5)
    for M, N, K in [(1, 777, 1000), (200, 300, 700)]:
        xg, xc = rand_packed(rng, M, K)
        wg, wc = rand_packed(rng, N, K)
        alpha = rng.standard_normal(N).astype(np.float32)
        xd, wd = to_dev_words(xg), to_dev_words(wg)
        assert np.array_equal(bnn.gemm_u64(xd, wd, K).cpu().numpy(), oracle.gemm_i32(xc, wc, K))
        assert_scaled_equal(bnn.gemm_u64_scaled(xd, wd, torch.from_numpy(alpha).to(DEV), K)
                            .cpu().numpy(), oracle.gemm_scaled(xc, wc, alpha, K))
        assert np.array_equal(words_np(bnn.gemm_sign_repack(xd, wd, K)),
                              oracle.sign_repack(xc, wc, K))


@pytest.mark.parametrize("M", [1, 64])
def test_k_zero_and_empty_products(M):
    for algo in ALGOS:
        xd = torch.empty(M, 0, dtype=torch.int64, device=DEV)
        wd = torch.empty(1000, 0, dtype=torch.int64, device=DEV)
        y = bnn.gemm_ex(xd, wd, 0, bnn.EPI_I32, algo)
        assert y.shape == (M, 1000) and not y.any()
        a = torch.randn(1000, device=DEV)
        assert not bnn.gemm_ex(xd, wd, 0, bnn.EPI_SCALED, algo, alpha=a).any()
        p = words_np(bnn.gemm_ex(xd, wd, 0, bnn.EPI_REPACK, algo))
        assert np.all(p[:, :15] == np.uint64(0xFFFFFFFFFFFFFFFF))
        assert np.all(p[:, 15] == np.uint64(0x000000FFFFFFFFFF))
    e = torch.empty(0, 2, dtype=torch.int64, device=DEV)
    w = torch.zeros(3, 2, dtype=torch.int64, device=DEV)
    assert bnn.gemm_u64(e, w, 100).shape == (0, 3)
    assert bnn.gemm_u64(w, e, 100).shape == (3, 0)


def test_large_k():
    # K ~ 1M bits: long K loops, int32 range, last word 3 bits wide
    rng = np.random.default_rng(9)
    M, N, K = 3, 70, 1_000_003
    xg, xc = rand_packed(rng, M, K)
    wg, wc = rand_packed(rng, N, K)
    ref = oracle.gemm_i32(xc, wc, K)
    for algo in ALGOS:
        got = bnn.gemm_ex(to_dev_words(xg), to_dev_words(wg), K, bnn.EPI_I32, algo).cpu().numpy()
        assert np.array_equal(got, ref)


def test_unaligned_16b_operands_use_narrow_loads():
    # 8-byte aligned but not 16-byte aligned operands (views starting at word 1)
    rng = np.random.default_rng(10)
    M, N, K = 2, 100, 256
    xg, xc = rand_packed(rng, M, K)
    wg, wc = rand_packed(rng, N, K)
    xbig = to_dev_words(np.concatenate([np.zeros(1, np.uint64), xg.ravel()]))
    wbig = to_dev_words(np.concatenate([np.zeros(1, np.uint64), wg.ravel()]))
    xd = xbig[1:].view(M, oracle.words(K))
    wd = wbig[1:].view(N, oracle.words(K))
    assert xd.data_ptr() % 16 == 8
    got = bnn.gemm_ex(xd, wd, K, bnn.EPI_I32, bnn.ALGO_GEMV).cpu().numpy()
    assert np.array_equal(got, oracle.gemm_i32(xc, wc, K))


def test_runs_on_a_side_stream():
    rng = np.random.default_rng(12)
    xg, xc = rand_packed(rng, 40, 300)
    wg, wc = rand_packed(rng, 50, 300)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = bnn.gemm_u64(to_dev_words(xg), to_dev_words(wg), 300)
    s.synchronize()
    assert np.array_equal(y.cpu().numpy(), oracle.gemm_i32(xc, wc, 300))


# ---------------------------------------------------------------------------
# bnn_gemm_sign_repack_thr: per-channel threshold and flip mask


def flags_of(mask: np.ndarray, n: int) -> np.ndarray:
    """Per-channel flags (uint8) from a packed mask: bit c%64 of word c/64."""
    bits = np.unpackbits(np.ascontiguousarray(mask, np.uint64).view(np.uint8), bitorder="little")
    return bits[:n].astype(np.uint8)


def rand_thr(rng, n, k):
    thr = rng.integers(-k - 3, k + 3, n).astype(np.int64)
    if n >= 6:
        thr[:6] = [-(2 ** 31), 2 ** 31 - 1, -k - 1, -k, k, k - 1]
    return thr.astype(np.int32)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("algo", ALGOS)
def test_repack_thr_parity(M, N, K, algo):
    say("repack_thr", M, N, K, "algo", algo)
    rng = np.random.default_rng(M * 7 + N * 1013 + K * 31 + 1)
    xg, xc = rand_packed(rng, M, K)
    wg, wc = rand_packed(rng, N, K)
    xd, wd = to_dev_words(xg), to_dev_words(wg)
    thr = rand_thr(rng, N, K)
    td = torch.from_numpy(thr).to(DEV)
    # flip mask with garbage past column N (it must be ignored)
    mask = rng.integers(0, 2 ** 64, size=oracle.words(N), dtype=np.uint64)
    got = words_np(bnn.gemm_sign_repack_thr(xd, wd, td, K, to_dev_words(mask[None])[0], algo))
    assert np.array_equal(got, oracle.sign_repack_thr(xc, wc, thr, K, flags_of(mask, N)))
    got = words_np(bnn.gemm_sign_repack_thr(xd, wd, td, K, None, algo))
    assert np.array_equal(got, oracle.sign_repack_thr(xc, wc, thr, K))
    zero = torch.zeros(N, dtype=torch.int32, device=DEV)
    got = words_np(bnn.gemm_sign_repack_thr(xd, wd, zero, K, None, algo))
    assert np.array_equal(got, oracle.sign_repack(xc, wc, K))


def test_repack_thr_extreme_k_on_matrix_cores():
    # K = 2^24, the matrix-core limit: dots of exactly +-K against thresholds
    # -K - 1, -K, K - 1, K (the fp32 bound is exact only after clamping)
    K = 2 ** 24
    rng = np.random.default_rng(14)
    _, x = rand_packed(rng, 2, K)
    w = np.stack([x[0], ~x[0], x[1], ~x[1]])
    thr = np.array([-K - 1, -K, K - 1, K], np.int32)
    ref = oracle.sign_repack_thr(x, w, thr, K)
    for algo in (bnn.ALGO_MFMA, bnn.ALGO_TILED, bnn.ALGO_GEMV):
        got = words_np(bnn.gemm_sign_repack_thr(to_dev_words(x), to_dev_words(w),
                                                torch.from_numpy(thr).to(DEV), K, None, algo))
        assert np.array_equal(got, ref), algo


def test_flip_words_matches_flags():
    rng = np.random.default_rng(15)
    for n in (1, 63, 64, 65, 1000):
        flags = rng.integers(0, 2, n).astype(np.uint8)
        got = words_np(bnn.flip_words(torch.from_numpy(flags).to(DEV))[None])[0]
        assert np.array_equal(flags_of(got, n), flags)
        assert got.shape == (oracle.words(n),)
        if n % 64:
            assert int(got[-1]) >> (n % 64) == 0


# ---------------------------------------------------------------------------
# the five workloads at full size


def test_workload_gemv_small():
    d = workloads.make("gemv_small")
    xp = bnn.pack_signs(d["x"].to(DEV))
    wp = bnn.pack_signs(d["w"].to(DEV))
    rx, rw = oracle.pack(d["x"].numpy()), oracle.pack(d["w"].numpy())
    assert np.array_equal(words_np(xp), rx) and np.array_equal(words_np(wp), rw)
    assert np.array_equal(bnn.gemm_u64(xp, wp, d["K"]).cpu().numpy(), oracle.gemm_i32(rx, rw, d["K"]))


def test_workload_gemv_4096():
    d = workloads.make("gemv_4096")
    xp = bnn.pack_signs(d["x"].to(DEV))
    wp = bnn.pack_signs(d["w"].to(DEV))
    rx, rw = oracle.pack(workloads.bf16_bits(d["x"])), oracle.pack(d["w"].numpy())
    assert np.array_equal(words_np(xp), rx) and np.array_equal(words_np(wp), rw)
    alpha = d["alpha"].numpy()
    got = bnn.gemm_u64_scaled(xp, wp, d["alpha"].to(DEV), d["K"]).cpu().numpy()
    assert_scaled_equal(got, oracle.gemm_scaled(rx, rw, alpha, d["K"]))


def test_workload_edge_1000():
    d = workloads.make("edge_1000")
    K = d["K"]
    xp = bnn.pack_signs(d["x"].to(DEV))
    wp = bnn.pack_signs(d["w"].to(DEV))
    rx, rw = oracle.pack(d["x"].numpy()), oracle.pack(d["w"].numpy())
    assert np.array_equal(words_np(xp), rx) and np.array_equal(words_np(wp), rw)
    assert np.array_equal(bnn.gemm_u64(xp, wp, K).cpu().numpy(), oracle.gemm_i32(rx, rw, K))
    alpha = d["alpha"].numpy()
    assert (alpha[::10] == 0).all()
    got = bnn.gemm_u64_scaled(xp, wp, d["alpha"].to(DEV), K).cpu().numpy()
    assert_scaled_equal(got, oracle.gemm_scaled(rx, rw, alpha, K))
    assert not got[:, ::10].any()
    # K = 0 companion call: every dot 0, every scaled output 0, every repacked bit -1
    e = torch.empty(64, 0, dtype=torch.int64, device=DEV)
    f = torch.empty(1000, 0, dtype=torch.int64, device=DEV)
    assert not bnn.gemm_u64(e, f, 0).any()
    assert not bnn.gemm_u64_scaled(e, f, d["alpha"].to(DEV), 0).any()


def _sample_pairs(rng, M, N, count):
    return rng.integers(0, M, count), rng.integers(0, N, count)


def test_workload_ffn_4096_every_output():
    # the benchmark's launch at its full size, every one of the 4096 x 11008
    # outputs against the oracle (about 10-20 s of host time)
    d = workloads.make("ffn_4096")
    K = d["K"]
    xp = bnn.pack_signs(d["x"].to(DEV))
    wp = bnn.pack_signs(d["w"].to(DEV))
    rx, rw = oracle.pack(workloads.bf16_bits(d["x"])), oracle.pack(d["w"].numpy())
    assert np.array_equal(words_np(xp), rx) and np.array_equal(words_np(wp), rw)
    y = bnn.gemm_u64_scaled(xp, wp, d["alpha"].to(DEV), K)
    say("ffn_4096: oracle on every output")
    assert_scaled_equal(y.cpu().numpy(), oracle.gemm_scaled(rx, rw, d["alpha"].numpy(), K))


def test_workload_chain_65536():
    # the four separate launches at the full size, every row of every stage
    # against the oracle's chain
    d = workloads.make("chain_65536")
    dims = d["dims"]
    x = d["x"]
    h = bnn.pack_signs(x.to(DEV))
    wps = [bnn.pack_signs(w.to(DEV)) for w in d["weights"]]
    h1 = bnn.gemm_sign_repack(h, wps[0], dims[0])
    h2 = bnn.gemm_sign_repack(h1, wps[1], dims[1])
    y = bnn.gemm_u64_scaled(h2, wps[2], d["alpha"].to(DEV), dims[2])
    final, hidden = oracle.chain(x.numpy(), [w.numpy() for w in d["weights"]],
                                 d["alpha"].numpy())
    assert np.array_equal(words_np(h), oracle.pack(x.numpy()))
    assert np.array_equal(words_np(h1), hidden[0])
    assert np.array_equal(words_np(h2), hidden[1])
    assert_scaled_equal(y.cpu().numpy(), final)


def test_workload_chain_65536_bn_folded():
    # the same chain with a BatchNorm after each hidden binary layer, folded
    # into per-channel thresholds and flips on the host
    from packed_xor_popcount_amd.fold import bn_fold
    d = workloads.make("chain_65536")
    dims = d["dims"]
    x = d["x"]
    rng = np.random.default_rng(56)
    params = []
    for i in range(2):
        n = d["weights"][i].shape[0]
        k = dims[i]
        gamma = rng.standard_normal(n)
        beta = rng.standard_normal(n)
        mean = rng.standard_normal(n) * np.sqrt(k)
        std = np.abs(rng.standard_normal(n)) + 0.5
        params.append(bn_fold(gamma, beta, mean, std, np.ones(n), k))
    h = bnn.pack_signs(x.to(DEV))
    wps = [bnn.pack_signs(w.to(DEV)) for w in d["weights"]]
    hs = []
    for i in range(2):
        thr, flip = params[i]
        fd = bnn.flip_words(torch.from_numpy(flip).to(DEV))
        h = bnn.gemm_sign_repack_thr(h, wps[i], torch.from_numpy(thr).to(DEV), dims[i], fd)
        hs.append(h)
    y = bnn.gemm_u64_scaled(h, wps[2], d["alpha"].to(DEV), dims[2])
    # every row against the oracle
    r = oracle.pack(x.numpy())
    for i in range(2):
        r = oracle.sign_repack_thr(r, oracle.pack(d["weights"][i].numpy()), params[i][0], dims[i],
                                   params[i][1])
        assert np.array_equal(words_np(hs[i]), r), i
    ref = oracle.gemm_scaled(r, oracle.pack(d["weights"][2].numpy()), d["alpha"].numpy(), dims[2])
    assert_scaled_equal(y.cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# bnn_gemv_act: activation packing fused into the weight-streaming product

ACT_SHAPES = [(1, 1, 1), (1, 256, 512), (1, 4096, 4096), (3, 100, 65), (8, 300, 1000),
              (9, 77, 129), (20, 64, 4095), (2, 130, 40000), (1, 50, 70001), (5, 1000, 0)]


@pytest.mark.parametrize("M,N,K", ACT_SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gemv_act_parity(M, N, K, dtype):
    say("gemv_act", M, N, K, dtype)
    c = workloads.random_case(seed=M * 31 + N * 7 + K, M=M, N=N, K=K, dist="normal",
                              zero_frac=0.01 if M * K >= 2 else 0.0, dtype=dtype)
    x, K = c["x"], c["K"]
    rng = np.random.default_rng(K + 1)
    wg, wc = rand_packed(rng, N, K)
    alpha = c["alpha"]
    xd, wd, ad = x.to(DEV), to_dev_words(wg), alpha.to(DEV)
    rx = oracle.pack(host_input(x), k=K) if M else np.zeros((0, oracle.words(K)), np.uint64)
    assert np.array_equal(bnn.gemv_act(xd, wd, K, bnn.EPI_I32).cpu().numpy(),
                          oracle.gemm_i32(rx, wc, K))
    assert_scaled_equal(bnn.gemv_act(xd, wd, K, bnn.EPI_SCALED, alpha=ad).cpu().numpy(),
                        oracle.gemm_scaled(rx, wc, alpha.numpy(), K))
    assert np.array_equal(words_np(bnn.gemv_act(xd, wd, K, bnn.EPI_REPACK)),
                          oracle.sign_repack(rx, wc, K))


@pytest.mark.parametrize("M", [2, 5, 8])
@pytest.mark.parametrize("K", [512, 4096])
@pytest.mark.parametrize("pad", [0, 1])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gemv_act_several_rows(M, K, pad, dtype):
    # the straight-line batch form with 2..8 rows: each row's words in LDS,
    # rows contiguous (pad 0) or with a padded stride that keeps every row
    # start 16-byte aligned (pad 1)
    N = 77 + 1000 * (K == 512)
    say("gemv_act rows", M, K, pad, dtype, N)
    esize = 4 if dtype == torch.float32 else 2
    ld = K + pad * (16 // esize)
    c = workloads.random_case(seed=M * 131 + K + pad, M=M, N=N, K=ld, dist="normal",
                              zero_frac=0.01, dtype=dtype)
    big = c["x"]
    rng = np.random.default_rng(M + K + pad)
    wg, wc = rand_packed(rng, N, K)
    alpha = c["alpha"][:N]
    xd = big.to(DEV)[:, :K]
    assert xd.stride(0) == ld and (ld * esize) % 16 == 0
    wd, ad = to_dev_words(wg), alpha.to(DEV)
    rx = oracle.pack(np.ascontiguousarray(host_input(big)[:, :K]))
    assert np.array_equal(bnn.gemv_act(xd, wd, K, bnn.EPI_I32).cpu().numpy(),
                          oracle.gemm_i32(rx, wc, K))
    assert_scaled_equal(bnn.gemv_act(xd, wd, K, bnn.EPI_SCALED, alpha=ad).cpu().numpy(),
                        oracle.gemm_scaled(rx, wc, alpha.numpy(), K))
    assert np.array_equal(words_np(bnn.gemv_act(xd, wd, K, bnn.EPI_REPACK)),
                          oracle.sign_repack(rx, wc, K))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gemv_act_strided_rows(dtype):
    # row stride 1003 elements (not a multiple of 16 bytes): guarded loads
    g = workloads.generator(31)
    big = workloads.normal(g, 4, 1003).to(dtype)
    x = big[:, :900]
    rng = np.random.default_rng(31)
    wg, wc = rand_packed(rng, 70, 900)
    rx = oracle.pack(np.ascontiguousarray(host_input(big)[:, :900]))
    got = bnn.gemv_act(big.to(DEV)[:, :900], to_dev_words(wg), 900, bnn.EPI_I32).cpu().numpy()
    assert np.array_equal(got, oracle.gemm_i32(rx, wc, 900))
    assert x.shape == (4, 900)


def test_gemv_act_workload_gemv_4096():
    # the benchmark's one-launch step: bf16 x packed in-kernel, alpha-scaled output
    d = workloads.make("gemv_4096")
    wp = bnn.pack_signs(d["w"].to(DEV))
    y = bnn.gemv_act(d["x"].to(DEV), wp, d["K"], bnn.EPI_SCALED, alpha=d["alpha"].to(DEV))
    rx, rw = oracle.pack(workloads.bf16_bits(d["x"])), oracle.pack(d["w"].numpy())
    assert_scaled_equal(y.cpu().numpy(), oracle.gemm_scaled(rx, rw, d["alpha"].numpy(), d["K"]))


@pytest.mark.parametrize("M,N,K", [(1, 20000, 4096), (3, 140000, 200), (2, 40000, 1000),
                                   (1, 70000, 130)])
def test_gemv_many_columns(M, N, K):
    # N beyond one wave of persistent blocks: the four-pass step and the
    # grid-stride loop of the GEMV kernel, packed and fused activations
    say("gemv many columns", M, N, K)
    c = workloads.random_case(seed=N + K, M=M, N=N, K=K, dist="normal", dtype=torch.bfloat16)
    rng = np.random.default_rng(N)
    wg, wc = rand_packed(rng, N, K)
    rx = oracle.pack(host_input(c["x"]))
    alpha = c["alpha"]
    xd, wd, ad = c["x"].to(DEV), to_dev_words(wg), alpha.to(DEV)
    xpd = to_dev_words(rx)
    ref = oracle.gemm_i32(rx, wc, K)
    refs = oracle.gemm_scaled(rx, wc, alpha.numpy(), K)
    refp = oracle.sign_repack(rx, wc, K)
    assert np.array_equal(bnn.gemm_ex(xpd, wd, K, bnn.EPI_I32, bnn.ALGO_GEMV).cpu().numpy(), ref)
    assert_scaled_equal(bnn.gemm_ex(xpd, wd, K, bnn.EPI_SCALED, bnn.ALGO_GEMV, alpha=ad)
                        .cpu().numpy(), refs)
    assert np.array_equal(words_np(bnn.gemm_ex(xpd, wd, K, bnn.EPI_REPACK, bnn.ALGO_GEMV)), refp)
    assert np.array_equal(bnn.gemv_act(xd, wd, K, bnn.EPI_I32).cpu().numpy(), ref)
    assert_scaled_equal(bnn.gemv_act(xd, wd, K, bnn.EPI_SCALED, alpha=ad).cpu().numpy(), refs)
    assert np.array_equal(words_np(bnn.gemv_act(xd, wd, K, bnn.EPI_REPACK)), refp)


@pytest.mark.parametrize("M,N,K,dtype", [(1, 150001, 4096, torch.bfloat16),
                                         (3, 150001, 4096, torch.float32),
                                         (2, 600007, 200, torch.bfloat16),
                                         (8, 600007, 200, torch.float32)])
def test_gemv_multi_step_blocks(M, N, K, dtype):
    # N beyond one step per persistent block: blocks of two or three steps
    # (the streaming form: each step's operands loaded one step ahead, pairs
    # of steps, an odd last step), real-valued and packed rows
    say("gemv multi-step", M, N, K, dtype)
    c = workloads.random_case(seed=N + K + M, M=M, N=N, K=K, dist="normal", dtype=dtype)
    rng = np.random.default_rng(N + M)
    wg, wc = rand_packed(rng, N, K)
    rx = oracle.pack(host_input(c["x"]))
    alpha = c["alpha"]
    xd, wd, ad = c["x"].to(DEV), to_dev_words(wg), alpha.to(DEV)
    xpd = to_dev_words(rx)
    ref = oracle.gemm_i32(rx, wc, K)
    refs = oracle.gemm_scaled(rx, wc, alpha.numpy(), K)
    refp = oracle.sign_repack(rx, wc, K)
    assert np.array_equal(bnn.gemv_act(xd, wd, K, bnn.EPI_I32).cpu().numpy(), ref)
    assert_scaled_equal(bnn.gemv_act(xd, wd, K, bnn.EPI_SCALED, alpha=ad).cpu().numpy(), refs)
    assert np.array_equal(words_np(bnn.gemv_act(xd, wd, K, bnn.EPI_REPACK)), refp)
    assert np.array_equal(bnn.gemm_u64(xpd, wd, K).cpu().numpy(), ref)
    assert_scaled_equal(bnn.gemm_u64_scaled(xpd, wd, ad, K).cpu().numpy(), refs)
