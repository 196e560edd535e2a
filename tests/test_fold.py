"""Host-side BatchNorm folding (packed_xor_popcount_amd.fold), checked against
a float64 BatchNorm evaluated on exact dots and projected to signs, through
the oracle's threshold repack ("Architecture Decision Record", Decision: BN
after the binary layers).  CPU only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from packed_xor_popcount_amd.fold import bn_fold
from tests.test_oracle_pins import np_unpack, rand_packed


def _bn_signs(d, gamma, beta, mean, std, alpha):
    z = gamma * (alpha * d - mean) / std + beta
    return np.where(z <= 0, -1.0, 1.0).astype(np.float32)


@pytest.mark.parametrize("seed,M,N,K", [(22, 9, 200, 333), (23, 4, 64, 64), (24, 3, 130, 7)])
def test_bn_fold_matches_float64_batchnorm(seed, M, N, K):
    rng = np.random.default_rng(seed)
    xp, wp = rand_packed(rng, M, K), rand_packed(rng, N, K)
    d = (np_unpack(xp, K) @ np_unpack(wp, K).T).astype(np.float64)
    gamma = rng.standard_normal(N) * 2
    gamma[:5] = 0.0                    # zero slope: a constant sign
    beta = rng.standard_normal(N) * 3
    beta[:2] = [-1.0, 1.0]
    mean = rng.standard_normal(N) * K ** 0.5 * 2
    mean[5:8] = [10 * K, -10 * K, 0.0]  # thresholds far outside [-K, K]
    std = np.abs(rng.standard_normal(N)) + 0.1
    alpha = np.abs(rng.standard_normal(N)) + 0.05
    alpha[8:12] *= -1                  # negative scales flip the slope too
    thr, flip = bn_fold(gamma, beta, mean, std, alpha, K)
    assert thr.dtype == np.int32 and flip.dtype == np.uint8
    assert thr.min() >= -K - 1 and thr.max() <= K
    ref = oracle.pack(_bn_signs(d, gamma, beta, mean, std, alpha))
    assert np.array_equal(oracle.sign_repack_thr(xp, wp, thr, K, flip), ref)


def test_bn_fold_exact_boundaries():
    # tau lands exactly on an integer dot: z = 0 there projects to -1, so the
    # threshold must include it (s > 0) or exclude it from the +1 side (s < 0)
    K = 10
    d = np.arange(-K, K + 1, 2, dtype=np.float64)[None, :]
    for g in (1.0, -1.0):
        thr, flip = bn_fold([g], [0.0], [4.0], [1.0], [1.0], K)
        bits = (d <= thr[0]) ^ bool(flip[0])
        z = g * (d - 4.0)
        assert np.array_equal(bits, z <= 0), g


def test_bn_fold_rejects_bad_parameters():
    with pytest.raises(ValueError):
        bn_fold([1.0], [0.0], [0.0], [0.0], [1.0], 8)
    with pytest.raises(ValueError):
        bn_fold([1.0], [0.0], [0.0], [1.0], [0.0], 8)
