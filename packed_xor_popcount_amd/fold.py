"""Folding a per-channel BatchNorm into the threshold repack.

"Architecture Decision Record", Decision: the binary layers are followed by
BatchNorm.  Between two binary layers the BatchNorm output only feeds the
next layer's sign projection, so it collapses into one integer comparison
per channel on the layer's exact dot d in [-K, K]:

    z(d) = gamma * (alpha * d - mean) / std + beta,  projected to -1 iff z <= 0.

With slope s = gamma * alpha / std and tau = (mean - beta * std / gamma) / alpha:

* s > 0: z <= 0 iff d <= tau iff d <= floor(tau)          -> thr = floor(tau)
* s < 0: z <= 0 iff d >= tau iff not (d <= ceil(tau) - 1) -> thr = ceil(tau) - 1, flip
* s = 0: z = beta for every d                             -> thr = K, flip iff beta > 0

These are the (thr, flip) operands of ``gemm_sign_repack_thr``.  This is
model-conversion code run once on the host (float64 numpy), not part of the
product path.  Where tau falls on an integer to within float64 rounding the
comparison at that single d is as float64 decides it.
"""
from __future__ import annotations

import numpy as np


def bn_fold(gamma, beta, mean, std, alpha, K: int):
    """Return ``(thr int32 (N,), flip uint8 (N,))`` for per-channel BatchNorm
    parameters (``std`` = sqrt(running_var + eps)) and per-channel weight
    scales ``alpha`` (ones for an unscaled layer) of a layer with K inputs.
    Thresholds are clamped to [-K - 1, K] (every dot lies in [-K, K])."""
    g = np.asarray(gamma, np.float64)
    b = np.asarray(beta, np.float64)
    mu = np.asarray(mean, np.float64)
    sd = np.asarray(std, np.float64)
    a = np.asarray(alpha, np.float64)
    g, b, mu, sd, a = np.broadcast_arrays(g, b, mu, sd, a)
    if np.any(sd <= 0) or np.any(a == 0):
        raise ValueError("std must be positive and alpha non-zero")
    s = g * a / sd
    thr = np.zeros(g.shape, np.float64)
    flip = np.zeros(g.shape, np.uint8)
    pos, neg, zero = s > 0, s < 0, s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        tau = (mu - b * sd / g) / a
    thr[pos] = np.floor(tau[pos])
    thr[neg] = np.ceil(tau[neg]) - 1
    flip[neg] = 1
    thr[zero] = K
    flip[zero] = (b[zero] > 0).astype(np.uint8)
    thr = np.clip(thr, -K - 1, K).astype(np.int32)
    return thr, flip
