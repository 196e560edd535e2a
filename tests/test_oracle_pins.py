"""Pins for the CPU oracle: checks of the oracle against what the pages and
the mathematics fix, none of which re-types the oracle's own formula.

Sources: "Binary Math Effectiveness -- why / how / when", section 1 (encoding
table, the identity <x,w> = n - 2d and its XNOR form 2a - n, the edge-case
table) and section 2.1 (ceil(K/64) words per row).

Pins (each is a function of the oracle object so that the mutation test at
the bottom can run them against deliberately broken copies):
  worked examples     hand-worked words and dots (tests/golden)
  projection tables   fp32 / bf16 truth tables (tests/golden)
  repack examples     dots -> packed sign words (tests/golden)
  scaled examples     alpha * dot, alpha = 0 -> 0 (tests/golden)
  identity triple     oracle == n - 2 popcount(xor) == 2 popcount(xnor) - n,
                      computed here with numpy bit operations
  brute force         every pair of +-1 vectors for n = 0..10
  special cases       x = w -> n, x = -w -> -n, |dot| <= n, dot = n (mod 2)
  padding             garbage pad bits change nothing; packed pads are 0
  library witness     float64 torch.matmul of independently unpacked +-1
                      matrices, at the shapes of every workload
  scaled closed form  numpy fp32 product of the integer result and alpha
  repack composition  sign_repack == pack(float(gemm))
  chain               numpy +-1 forward pass of the whole layer chain
"""
from __future__ import annotations

import itertools
import types

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _golden

# --------------------------------------------------------------------------
# Independent helpers (numpy only; no oracle code).


def np_unpack(p: np.ndarray, k: int) -> np.ndarray:
    """+-1 int64 (rows, k) from packed words, via numpy's bit unpacking:
    little-endian words, least significant bit first."""
    p = np.ascontiguousarray(p, dtype=np.uint64)
    rows = p.shape[0]
    bits = np.unpackbits(p.view(np.uint8).reshape(rows, -1), axis=1, bitorder="little")[:, :k]
    return 1 - 2 * bits.astype(np.int64)


def np_tail_mask(k: int) -> np.ndarray:
    kw = (k + 63) // 64
    m = np.full(kw, np.uint64(0xFFFFFFFFFFFFFFFF), dtype=np.uint64)
    if kw and k % 64:
        m[-1] = np.uint64((1 << (k % 64)) - 1)
    return m


def garbage_pads(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """Random words with bits only in pad positions (index >= k of a row)."""
    kw = (k + 63) // 64
    out = np.zeros((rows, kw), dtype=np.uint64)
    if kw and k % 64:
        rnd = rng.integers(0, 2 ** 63, size=rows, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
        out[:, -1] = rnd & ~np.uint64((1 << (k % 64)) - 1)
    return out


def rand_packed(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """Random packed rows with zero pad bits."""
    kw = (k + 63) // 64
    p = rng.integers(0, 2 ** 64, size=(rows, kw), dtype=np.uint64)
    return p & np_tail_mask(k)[None, :] if kw else p


# --------------------------------------------------------------------------
# Pins as functions of the oracle object.


def pin_worked_examples(o):
    for n, xs, ws, xw, ww, d, dot in _golden.worked_examples():
        assert n - 2 * d == dot  # the fixture itself is consistent
        x, w = _golden.signs_to_f32(xs), _golden.signs_to_f32(ws)
        xp, wp = o.pack(x), o.pack(w)
        assert xp.shape == (1, o.words(n))
        assert [int(v) for v in xp[0]] == xw, (n, xs)
        assert [int(v) for v in wp[0]] == ww, (n, ws)
        assert int(o.gemm_i32(xp, wp, n)[0, 0]) == dot, (n, xs, ws)


def pin_projection_tables(o):
    for bits, desc, bit in _golden.projection_f32():
        v = np.array([[bits]], dtype=np.uint32).view(np.float32)
        got = int(o.pack(v)[0, 0])
        assert got == bit, ("fp32", desc, got)
        assert o.sign_f32(float(v[0, 0])) == (1 - 2 * bit), ("fp32 sign", desc)
    for bits, desc, bit in _golden.projection_bf16():
        v = np.array([[bits]], dtype=np.uint16)
        got = int(o.pack(v)[0, 0])
        assert got == bit, ("bf16", desc, got)
        assert o.sign_bf16(bits) == (1 - 2 * bit), ("bf16 sign", desc)


def pin_repack_examples(o):
    for k, dots, words in _golden.repack_examples():
        x, w = _golden.pair_rows_for_dots(k, dots)
        xp, wp = o.pack(x), o.pack(w)
        assert [int(v) for v in o.gemm_i32(xp, wp, k)[0]] == dots
        got = o.sign_repack(xp, wp, k)
        assert got.shape == (1, o.words(len(dots)))
        assert [int(v) for v in got[0]] == words, (k, dots)


def pin_scaled_examples(o):
    for dot, alpha, exp in _golden.scaled_examples():
        k = abs(dot) if dot != 0 else 2
        x, w = _golden.pair_rows_for_dots(k, [dot])
        y = o.gemm_scaled(o.pack(x), o.pack(w), np.array([alpha], np.float32), k)
        assert y.dtype == np.float32 and y[0, 0] == exp, (dot, alpha, y[0, 0])


def pin_identity_triple(o, seed=11):
    rng = np.random.default_rng(seed)
    for k in (1, 5, 63, 64, 65, 100, 127, 128, 129, 1000):
        M, N = 5, 7
        xp, wp = rand_packed(rng, M, k), rand_packed(rng, N, k)
        mask = np_tail_mask(k)
        xr = (xp[:, None, :] ^ wp[None, :, :]) & mask
        d = np.bitwise_count(xr).sum(axis=2).astype(np.int64)
        a = np.bitwise_count(~(xp[:, None, :] ^ wp[None, :, :]) & mask).sum(axis=2).astype(np.int64)
        y = o.gemm_i32(xp, wp, k).astype(np.int64)
        assert np.array_equal(y, k - 2 * d), k
        assert np.array_equal(y, 2 * a - k), k


def pin_brute_force(o, nmax=10):
    for n in range(0, nmax + 1):
        codes = np.arange(2 ** n, dtype=np.int64)
        # all sign vectors of length n: element i is -1 when bit i of the code is 1
        S = 1 - 2 * ((codes[:, None] >> np.arange(n)[None, :]) & 1)
        expect = S @ S.T
        P = o.pack(S.astype(np.float32))
        got = o.gemm_i32(P, P, n).astype(np.int64)
        assert np.array_equal(got, expect), n
        if n <= 3:  # textbook loops for the smallest sizes
            for xi, wi in itertools.product(range(2 ** n), repeat=2):
                assert got[xi, wi] == sum(int(S[xi, t]) * int(S[wi, t]) for t in range(n))


def pin_special_cases(o, seed=12):
    rng = np.random.default_rng(seed)
    for k in (0, 1, 64, 65, 333):
        xp = rand_packed(rng, 6, k)
        neg = (~xp) & np_tail_mask(k)[None, :] if k else xp
        same = o.gemm_i32(xp, xp, k)
        assert np.all(np.diag(same) == k)
        assert np.all(np.diag(o.gemm_i32(xp, neg, k)) == -k)
        wp = rand_packed(rng, 9, k)
        y = o.gemm_i32(xp, wp, k).astype(np.int64)
        assert np.all(np.abs(y) <= k) and np.all((y - k) % 2 == 0)
        if k == 0:
            assert y.shape == (6, 9) and not y.any()
            alpha = rng.standard_normal(9).astype(np.float32)
            assert not o.gemm_scaled(xp, wp, alpha, 0).any()
            r = o.sign_repack(xp, wp, 0)
            assert np.all(r == np.uint64((1 << 9) - 1))  # 0 <= 0 -> -1 everywhere
        alpha0 = np.zeros(9, np.float32)
        assert not o.gemm_scaled(xp, wp, alpha0, k).any()


def pin_padding(o, seed=13):
    rng = np.random.default_rng(seed)
    for k in (1, 63, 65, 100, 1000):
        xp, wp = rand_packed(rng, 4, k), rand_packed(rng, 6, k)
        gx, gw = xp | garbage_pads(rng, 4, k), wp | garbage_pads(rng, 6, k)
        assert np.array_equal(o.gemm_i32(xp, wp, k), o.gemm_i32(gx, gw, k))
        assert np.array_equal(o.sign_repack(xp, wp, k), o.sign_repack(gx, gw, k))
        src = rng.standard_normal((3, k)).astype(np.float32)
        p = o.pack(src)
        assert not np.any(p & ~np_tail_mask(k)[None, :])


def pin_library_witness(o, M, N, K, seed, nrows=None):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    wf = rng.standard_normal((N, K)).astype(np.float32)
    xp, wp = o.pack(xf), o.pack(wf)
    if nrows is not None and nrows < M:
        rows = np.sort(rng.choice(M, nrows, replace=False))
        xp, xf = xp[rows], xf[rows]
    xs = torch.from_numpy(np_unpack(xp, K).astype(np.float64))
    ws = torch.from_numpy(np_unpack(wp, K).astype(np.float64))
    ref = torch.matmul(xs, ws.T).numpy()
    got = o.gemm_i32(xp, wp, K)
    assert np.array_equal(got.astype(np.float64), ref), (M, N, K)
    # and the unpacked operands are the sign projection of the floats
    assert np.array_equal(np_unpack(xp, K), np.where(xf > 0, 1, -1))


def pin_scaled_closed_form(o, seed=14):
    rng = np.random.default_rng(seed)
    for M, N, K in ((3, 17, 70), (9, 5, 200), (1, 64, 4096)):
        xp, wp = rand_packed(rng, M, K), rand_packed(rng, N, K)
        alpha = (rng.standard_normal(N) * 10).astype(np.float32)
        alpha[::4] = 0.0
        y = o.gemm_i32(xp, wp, K)
        ref = y.astype(np.float32) * alpha[None, :]  # one fp32 multiply (numpy)
        got = o.gemm_scaled(xp, wp, alpha, K)
        assert got.dtype == np.float32
        assert np.array_equal(got.view(np.uint32)[ref != 0], ref.view(np.uint32)[ref != 0])
        assert np.all(got[ref == 0] == 0)


def pin_repack_composition(o, seed=15):
    rng = np.random.default_rng(seed)
    for M, N, K in ((4, 1, 10), (3, 63, 64), (5, 64, 65), (2, 65, 130), (7, 200, 333), (2, 0, 5)):
        xp, wp = rand_packed(rng, M, K), rand_packed(rng, N, K)
        y = o.gemm_i32(xp, wp, K).astype(np.float32)
        got = o.sign_repack(xp, wp, K)
        assert got.shape == (M, o.words(N))
        if N:
            assert np.array_equal(got, o.pack(y))


def pin_chain(o, seed=16):
    rng = np.random.default_rng(seed)
    dims = (96, 70, 130, 33)
    x = rng.standard_normal((11, dims[0])).astype(np.float32)
    ws = [rng.standard_normal((dims[i + 1], dims[i])).astype(np.float32) for i in range(3)]
    alpha = np.abs(rng.standard_normal(dims[-1])).astype(np.float32)
    alpha[3] = 0.0
    final, hidden = o.chain(x, ws, alpha)
    # numpy forward pass on +-1 integers, straight from the definitions
    h = np.where(x > 0, 1, -1).astype(np.int64)
    for i, w in enumerate(ws):
        s = h @ np.where(w > 0, 1, -1).astype(np.int64).T
        if i < 2:
            assert np.array_equal(np_unpack(hidden[i], dims[i + 1]), np.where(s > 0, 1, -1))
            h = np.where(s > 0, 1, -1)
        else:
            ref = s.astype(np.float32) * alpha[None, :]
            assert np.array_equal(final[ref != 0], ref[ref != 0]) and np.all(final[ref == 0] == 0)


def pin_dot_pairs(o, seed=17):
    rng = np.random.default_rng(seed)
    K = 777
    xp, wp = rand_packed(rng, 20, K), rand_packed(rng, 30, K)
    mi, ni = rng.integers(0, 20, 50), rng.integers(0, 30, 50)
    full = o.gemm_i32(xp, wp, K)
    assert np.array_equal(o.dot_pairs(xp, wp, K, mi, ni), full[mi, ni])


# --------------------------------------------------------------------------
# The pins against the real oracle.


def test_words_closed_form():
    for k in (0, 1, 63, 64, 65, 127, 128, 129, 1000, 4096, 2 ** 31 - 1):
        assert oracle.words(k) == -(-k // 64)


def test_worked_examples():
    pin_worked_examples(oracle)


def test_projection_tables():
    pin_projection_tables(oracle)


def test_repack_examples():
    pin_repack_examples(oracle)


def test_scaled_examples():
    pin_scaled_examples(oracle)


def test_identity_triple():
    pin_identity_triple(oracle)


def test_brute_force():
    pin_brute_force(oracle)


def test_special_cases():
    pin_special_cases(oracle)


def test_padding():
    pin_padding(oracle)


@pytest.mark.parametrize("M,N,K,nrows", [
    (1, 256, 512, None),      # gemv_small
    (1, 4096, 4096, None),    # gemv_4096
    (64, 1000, 1000, None),   # edge_1000
    (4096, 11008, 4096, 3),   # ffn_4096, sampled rows
    (256, 256, 512, None),    # chain layer 1 (row slice)
    (256, 128, 256, None),    # chain layer 2
    (256, 64, 128, None),     # chain layer 3
])
def test_library_witness(M, N, K, nrows):
    pin_library_witness(oracle, M, N, K, seed=M + N + K, nrows=nrows)


def test_scaled_closed_form():
    pin_scaled_closed_form(oracle)


def test_repack_composition():
    pin_repack_composition(oracle)


def test_chain():
    pin_chain(oracle)


def test_dot_pairs():
    pin_dot_pairs(oracle)


def test_bf16_pack_matches_fp32_of_same_values():
    # bf16 -> fp32 widening is exact, so packing the bf16 bytes equals packing
    # their fp32 values (the workloads feed bf16 activations).
    g = workloads.generator(5)
    x = workloads.normal(g, 7, 300).to(torch.bfloat16)
    x[0, :10] = 0.0
    x[1, :10] = -0.0
    p16 = oracle.pack(workloads.bf16_bits(x))
    p32 = oracle.pack(x.to(torch.float32).numpy())
    assert np.array_equal(p16, p32)


def test_pack_row_stride():
    rng = np.random.default_rng(3)
    src = rng.standard_normal((5, 150)).astype(np.float32)
    assert np.array_equal(oracle.pack(src, k=100), oracle.pack(np.ascontiguousarray(src[:, :100])))


def test_threads_do_not_change_results():
    rng = np.random.default_rng(4)
    xp, wp = rand_packed(rng, 37, 300), rand_packed(rng, 41, 300)
    a = oracle.gemm_i32(xp, wp, 300, nthreads=1)
    b = oracle.gemm_i32(xp, wp, 300, nthreads=7)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("k", [0, 1, 63, 64, 65, 1000, 4096])
def test_unpack_round_trip_ignores_pad_bits(k):
    """oracle.unpack against numpy's own bit unpacking ("Binary Math
    Effectiveness", section 1 encoding table: bit 0 is +1, bit 1 is -1; pad
    bits past the logical n are not elements), with garbage pad bits."""
    rng = np.random.default_rng(100 + k)
    p = rand_packed(rng, 9, k)
    got = oracle.unpack(p | garbage_pads(rng, 9, k), k)
    assert got.dtype == np.int8 and got.shape == (9, k)
    assert np.array_equal(got.astype(np.int64), np_unpack(p, k))
    # pack(unpack) is the identity on pad-free words
    if k:
        assert np.array_equal(oracle.pack(got.astype(np.float32), k), p)


def test_unpack_worked_example():
    """Word 0b...1101 with K = 4: elements 0, 2, 3 are -1 and element 1 is +1
    (bit k of word 0 is element k, least significant bit first)."""
    p = np.array([[0b1101 | (0xF0 << 56)]], dtype=np.uint64)
    assert oracle.unpack(p, 4).tolist() == [[-1, 1, -1, -1]]


# --------------------------------------------------------------------------
# Mutation check: each plausible mistake planted in a copy of the oracle (on
# the CPU) must fail at least one pin.


def _mutant(**over):
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in (
        "words", "pack", "unpack", "gemm_i32", "gemm_scaled", "sign_repack", "dot_pairs",
        "chain", "sign_f32", "sign_bf16", "sign_repack_thr", "dot_signw_bf16")})
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _msb_first(p):
    out = np.zeros_like(p)
    for b in range(64):
        out |= ((p >> np.uint64(b)) & np.uint64(1)) << np.uint64(63 - b)
    return out


def _mutants():
    o = oracle
    yield "bit order msb-first", _mutant(pack=lambda s, k=None: _msb_first(o.pack(s, k)))
    yield "encoding flipped", _mutant(
        pack=lambda s, k=None: (~o.pack(s, k)) & np.stack(
            [np_tail_mask(np.asarray(s).shape[1] if k is None else k)] * np.asarray(s).shape[0]))
    yield "pads counted", _mutant(
        gemm_i32=lambda xp, wp, k, nthreads=0: o.gemm_i32(xp, wp, k) + (64 * o.words(k) - k))
    yield "sign of identity", _mutant(gemm_i32=lambda xp, wp, k, nthreads=0: -o.gemm_i32(xp, wp, k))
    yield "n - d instead of n - 2d", _mutant(
        gemm_i32=lambda xp, wp, k, nthreads=0: ((o.gemm_i32(xp, wp, k) + k) // 2).astype(np.int32))
    yield "tail word dropped", _mutant(
        gemm_i32=lambda xp, wp, k, nthreads=0: o.gemm_i32(
            np.ascontiguousarray(xp[:, : k // 64]), np.ascontiguousarray(wp[:, : k // 64]),
            64 * (k // 64)))
    yield "alpha by row", _mutant(
        gemm_scaled=lambda xp, wp, a, k, nthreads=0: o.gemm_i32(xp, wp, k).astype(np.float32)
        * np.resize(a, xp.shape[0])[:, None])
    yield "repack threshold < 0", _mutant(
        sign_repack=lambda xp, wp, k, nthreads=0: o.pack(o.gemm_i32(xp, wp, k).astype(np.float32) + 0.5)
        if wp.shape[0] else o.sign_repack(xp, wp, k))
    yield "zero projects to +1", _mutant(
        pack=lambda s, k=None: o.pack(np.where(np.asarray(s).view(np.float32) == 0, 1.0, s)
                                      .astype(np.float32), k)
        if np.asarray(s).dtype == np.float32 else o.pack(s, k))
    yield "NaN projects to +1", _mutant(
        pack=lambda s, k=None: o.pack(np.where(np.isnan(np.asarray(s)), 1.0, s).astype(np.float32), k)
        if np.asarray(s).dtype == np.float32 else o.pack(s, k))


_QUICK_PINS = [pin_worked_examples, pin_projection_tables, pin_repack_examples, pin_scaled_examples,
               pin_identity_triple, lambda o: pin_brute_force(o, 6), pin_special_cases, pin_padding,
               pin_scaled_closed_form, pin_repack_composition]


@pytest.mark.parametrize("name,mut", list(_mutants()), ids=[n for n, _ in _mutants()])
def test_pins_catch_planted_mistake(name, mut):
    failures = 0
    for pin in _QUICK_PINS:
        try:
            pin(mut)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, f"no pin catches the planted mistake: {name}"


# --------------------------------------------------------------------------
# Threshold repack ("Architecture Decision Record", Decision: "BN after
# binary"): bit = (dot <= thr[n]) xor flip[n].


def pin_repack_thr(o, seed=21):
    rng = np.random.default_rng(seed)
    for M, N, K in ((3, 70, 100), (5, 64, 65), (2, 130, 1000), (4, 1, 7)):
        xp, wp = rand_packed(rng, M, K), rand_packed(rng, N, K)
        # reduces to the plain projection rule at thr = 0, no flips
        assert np.array_equal(o.sign_repack_thr(xp, wp, np.zeros(N, np.int32), K),
                              o.sign_repack(xp, wp, K))
        # brute force against numpy dots of independently unpacked operands
        d = np_unpack(xp, K) @ np_unpack(wp, K).T
        thr = rng.integers(-K - 2, K + 2, N).astype(np.int32)
        flip = rng.integers(0, 2, N).astype(np.uint8)
        bits = (d <= thr[None, :]) ^ (flip[None, :] == 1)
        ref = o.pack(np.where(bits, -1.0, 1.0).astype(np.float32))
        assert np.array_equal(o.sign_repack_thr(xp, wp, thr, K, flip), ref)
        # extremes: every dot is in [-K, K]
        allm = o.sign_repack_thr(xp, wp, np.full(N, K, np.int32), K)
        assert np.array_equal(allm, o.pack(-np.ones((M, N), np.float32)))
        none = o.sign_repack_thr(xp, wp, np.full(N, -K - 1, np.int32), K)
        assert not none.any()


def test_repack_thr():
    pin_repack_thr(oracle)


def test_pins_catch_threshold_mistakes():
    o = oracle
    bad = [
        _mutant(sign_repack_thr=lambda xp, wp, t, k, flip=None, nthreads=0:
                o.sign_repack_thr(xp, wp, np.asarray(t, np.int32) - 1, k, flip)),   # "<" for "<="
        _mutant(sign_repack_thr=lambda xp, wp, t, k, flip=None, nthreads=0:
                o.sign_repack_thr(xp, wp, t, k, None)),                            # flip ignored
    ]
    for m in bad:
        with pytest.raises(AssertionError):
            pin_repack_thr(m)


# --------------------------------------------------------------------------
# Real-valued bf16 activations times packed sign weights (binary_nn README,
# "Binary Regression" / "Triton Kernel Benchmark"): s = sum_k x[k] w_n[k].


def bf16_of(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values that bf16 holds exactly (checked)."""
    f = np.asarray(v, dtype=np.float32)
    b = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << np.uint32(16)).view(np.float32), f)
    return b


def bf16_value(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32) \
        .astype(np.float64)


def rand_bf16(rng, rows, k):
    """N(0,1) values rounded to bf16 by truncation (any bf16 value will do)."""
    f = rng.standard_normal((rows, k)).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def pin_signw_examples(o):
    for x, signs, exp in _golden.signw_examples():
        k = x.size
        wp = o.pack(_golden.signs_to_f32(signs)) if k else np.zeros((1, 0), np.uint64)
        got = o.dot_signw_bf16(bf16_of(x).reshape(1, -1), wp, k)
        assert got.shape == (1, 1) and got[0, 0] == exp, (x, signs, got)


def pin_signw_library_witness(o, seed=31):
    # numpy float64 matmul of the bf16 values with independently unpacked
    # +-1 weights; both sums are exact in double for these inputs (8-bit
    # mantissas, exponents within 2^-20 .. 2^4, at most 2^11 terms)
    rng = np.random.default_rng(seed)
    for k in (1, 5, 63, 64, 65, 200, 1000, 2000):
        M, N = 4, 9
        xb = rand_bf16(rng, M, k)
        xv = bf16_value(xb)
        xv[np.abs(xv) < 2.0 ** -20] = 0.0
        xb = bf16_of(xv)
        wp = rand_packed(rng, N, k)
        ref = xv @ np_unpack(wp, k).T.astype(np.float64)
        assert np.array_equal(o.dot_signw_bf16(xb, wp, k), ref), k


def pin_signw_one_hot(o, seed=32):
    # x = e_k reads weight element k alone: bit order, word boundaries, pads
    rng = np.random.default_rng(seed)
    k = 130
    wp = rand_packed(rng, 5, k)
    garbage = wp | garbage_pads(rng, 5, k)
    eye = bf16_of(np.eye(k))
    ref = np_unpack(wp, k).T.astype(np.float64)     # [k][n]
    assert np.array_equal(o.dot_signw_bf16(eye, wp, k), ref)
    assert np.array_equal(o.dot_signw_bf16(eye, garbage, k), ref)


def pin_signw_binary_reduction(o, seed=33):
    # +-1 activations reduce it to the integer binary product of the packed
    # signs, i.e. K - 2 popcount(x xor w) computed here with numpy bit ops
    rng = np.random.default_rng(seed)
    for k in (1, 64, 100, 777):
        xp, wp = rand_packed(rng, 3, k), rand_packed(rng, 6, k)
        xv = np_unpack(xp, k).astype(np.float64)
        mask = np_tail_mask(k)
        d = np.bitwise_count((xp[:, None, :] ^ wp[None, :, :]) & mask).sum(axis=2).astype(np.int64)
        assert np.array_equal(o.dot_signw_bf16(bf16_of(xv), wp, k), (k - 2 * d).astype(np.float64))


def pin_signw_strided(o, seed=34):
    # rows read with their stride; columns past k are never read
    rng = np.random.default_rng(seed)
    big = rand_bf16(rng, 3, 90)
    wp = rand_packed(rng, 4, 70)
    ref = o.dot_signw_bf16(np.ascontiguousarray(big[:, :70]), wp, 70)
    assert np.array_equal(o.dot_signw_bf16(big, wp, 70), ref)
    poisoned = big.copy()
    poisoned[:, 70:] = 0x7FC0  # NaN past k
    assert np.array_equal(o.dot_signw_bf16(poisoned, wp, 70), ref)


_SIGNW_PINS = [pin_signw_examples, pin_signw_library_witness, pin_signw_one_hot,
               pin_signw_binary_reduction, pin_signw_strided]


@pytest.mark.parametrize("pin", _SIGNW_PINS, ids=[p.__name__ for p in _SIGNW_PINS])
def test_signw_pins(pin):
    pin(oracle)


def _msb_first_words(p):
    return _msb_first(np.ascontiguousarray(p, np.uint64))


def _signw_zero_columns(x, k, keep):
    """Copy of x (bf16 bits) with columns keep .. k-1 set to +0."""
    x = np.array(x, dtype=np.uint16, copy=True)
    x[:, keep:k] = 0
    return x


def test_signw_pins_catch_planted_mistakes():
    o = oracle

    def kk(x, k):
        return np.asarray(x).shape[1] if k is None else k

    mutants = {
        "weights negated": lambda x, wp, k=None, nthreads=0: -o.dot_signw_bf16(x, wp, k),
        "bit order msb-first": lambda x, wp, k=None, nthreads=0: o.dot_signw_bf16(
            x, _msb_first_words(wp), k),
        "last element dropped": lambda x, wp, k=None, nthreads=0: o.dot_signw_bf16(
            _signw_zero_columns(x, kk(x, k), max(kk(x, k) - 1, 0)), wp, k),
        "tail word dropped": lambda x, wp, k=None, nthreads=0: o.dot_signw_bf16(
            _signw_zero_columns(x, kk(x, k), 64 * (kk(x, k) // 64)), wp, k),
        "first row for all": lambda x, wp, k=None, nthreads=0: o.dot_signw_bf16(
            np.repeat(np.asarray(x)[:1], np.asarray(x).shape[0], axis=0), wp, k),
    }
    for name, f in mutants.items():
        m = _mutant(dot_signw_bf16=f)
        caught = 0
        for pin in _SIGNW_PINS:
            try:
                pin(m)
            except (AssertionError, ValueError):
                caught += 1
        assert caught, name
