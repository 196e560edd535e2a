"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds random-number generation and input preparation only: none
of the packed-binary arithmetic lives here, so the HIP path and the CPU
oracle can both be fed from it without sharing any of the method's code.

Every tensor is generated on the CPU with ``torch.Generator`` seeded per
workload, so the bytes are identical on every machine; callers copy them to
the GPU.  bf16 inputs are produced by rounding fp32 draws (round to nearest
even), and both sides read the same bf16 bytes.

The per-output-channel scale ``alpha[n] = mean_k |W[n, k]|`` is the absmean
scale that "Binary Math Effectiveness -- why / how / when", section 5, and the
balanced_ternary_engine README ("Features", absmean) describe; here it is an
input to the library, computed once in float64 and rounded once to fp32.

Workload shapes (seed = 1000 + index):
  1 gemv_small   M=1,     K=512,  N=256,   uniform(-1, 1) fp32, int32 out
  2 gemv_4096    M=1,     K=4096, N=4096,  W ~ N(0,1) fp32, x ~ N(0,1) bf16,
                                           alpha-scaled fp32 out
  3 edge_1000    M=64,    K=1000, N=1000,  uniform(-1, 1) fp32 with 1 % exact
                                           zeros (half +0, half -0), alpha = 0
                                           on every 10th channel, plus K = 0
  4 ffn_4096     M=4096,  K=4096, N=11008, X ~ N(0,1) bf16, W ~ N(0,1) fp32,
                                           alpha-scaled fp32 out
  5 chain_65536  M=65536, 512 -> 256 -> 128 -> 64, all ~ N(0,1) fp32; hidden
                                           layers sign -> repack, last layer
                                           alpha-scaled fp32
  6 signw_16384  M=16384, K=1024, N=1024,  X ~ N(0,1) bf16 kept real-valued,
                                           W ~ N(0,1) fp32 (sign-packed),
                                           alpha-scaled fp32 out: the largest
                                           packed-kernel shape of the binary_nn
                                           README ("Triton Kernel Benchmark")
"""
from __future__ import annotations

import torch

WORKLOADS = {
    "gemv_small": dict(index=1, M=1, K=512, N=256),
    "gemv_4096": dict(index=2, M=1, K=4096, N=4096),
    "edge_1000": dict(index=3, M=64, K=1000, N=1000),
    "ffn_4096": dict(index=4, M=4096, K=4096, N=11008),
    "chain_65536": dict(index=5, M=65536, dims=(512, 256, 128, 64)),
    "signw_16384": dict(index=6, M=16384, K=1024, N=1024),
}


def generator(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def uniform_pm1(g: torch.Generator, *shape) -> torch.Tensor:
    """fp32 drawn as 2*U[0,1) - 1."""
    return torch.rand(*shape, generator=g, dtype=torch.float32) * 2.0 - 1.0


def normal(g: torch.Generator, *shape) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def absmean_alpha(w: torch.Tensor) -> torch.Tensor:
    """alpha[n] = mean |W[n, :]| in float64, rounded once to fp32."""
    if w.shape[1] == 0:
        return torch.zeros(w.shape[0], dtype=torch.float32)
    return w.to(torch.float64).abs().mean(dim=1).to(torch.float32)


def plant_zeros(g: torch.Generator, t: torch.Tensor, frac: float = 0.01) -> torch.Tensor:
    """Set a seeded fraction of positions to exact zeros, half +0.0 and half
    -0.0 (both project to -1)."""
    t = t.clone()
    flat = t.view(-1)
    n = max(2, int(round(frac * flat.numel())))
    idx = torch.randperm(flat.numel(), generator=g)[:n]
    flat[idx[: n // 2]] = 0.0
    flat[idx[n // 2:]] = -0.0
    return t


def bf16_bits(t: torch.Tensor):
    """Raw 16-bit patterns of a bf16 tensor as a numpy uint16 array."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def make(name: str) -> dict:
    """Inputs of one named workload (CPU tensors)."""
    spec = WORKLOADS[name]
    g = generator(1000 + spec["index"])
    if name == "gemv_small":
        x = uniform_pm1(g, 1, 512)
        w = uniform_pm1(g, 256, 512)
        return dict(x=x, w=w, K=512)
    if name == "gemv_4096":
        w = normal(g, 4096, 4096)
        x = normal(g, 1, 4096).to(torch.bfloat16)
        return dict(x=x, w=w, alpha=absmean_alpha(w), K=4096)
    if name == "edge_1000":
        x = plant_zeros(g, uniform_pm1(g, 64, 1000))
        w = plant_zeros(g, uniform_pm1(g, 1000, 1000))
        alpha = absmean_alpha(w)
        alpha[0::10] = 0.0
        return dict(x=x, w=w, alpha=alpha, K=1000)
    if name == "ffn_4096":
        x = normal(g, 4096, 4096).to(torch.bfloat16)
        w = normal(g, 11008, 4096)
        return dict(x=x, w=w, alpha=absmean_alpha(w), K=4096)
    if name == "chain_65536":
        dims = spec["dims"]
        x = normal(g, spec["M"], dims[0])
        ws = [normal(g, dims[i + 1], dims[i]) for i in range(len(dims) - 1)]
        return dict(x=x, weights=ws, alpha=absmean_alpha(ws[-1]), dims=dims)
    if name == "signw_16384":
        x = normal(g, 16384, 1024).to(torch.bfloat16)
        w = normal(g, 1024, 1024)
        return dict(x=x, w=w, alpha=absmean_alpha(w), K=1024)
    raise KeyError(name)


def random_case(seed: int, M: int, N: int, K: int, dist: str = "uniform",
                zero_frac: float = 0.0, dtype: torch.dtype = torch.float32) -> dict:
    """A generic seeded case for property sweeps: X (M, K) and W (N, K) drawn
    uniform(-1, 1) or N(0, 1), optional exact zeros, X optionally bf16, and
    alpha = mean |W_row| with every 7th channel set to 0."""
    g = generator(seed)
    draw = uniform_pm1 if dist == "uniform" else normal
    x = draw(g, M, K)
    w = draw(g, N, K)
    if zero_frac > 0 and M * K >= 2:
        x = plant_zeros(g, x, zero_frac)
    if zero_frac > 0 and N * K >= 2:
        w = plant_zeros(g, w, zero_frac)
    alpha = absmean_alpha(w)
    alpha[0::7] = 0.0
    return dict(x=x.to(dtype), w=w, alpha=alpha, K=K)

