#!/usr/bin/env python3
"""Benchmark of the packed binary (XOR + popcount) hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Prints ONE JSON line.  A step is one pass of the hot path over one batch of
synthetic input, inputs already resident in HBM:

  gemv_4096 (default): one launch of bnn_gemv_act, which sign-packs the
      bf16 activation row (1 x 4096) inside the kernel and runs the
      alpha-scaled fp32 binary GEMV against a packed 4096 x 4096 weight
      matrix.  Step i reads weight copy i mod R from a ring of R = 256
      distinct copies (512 MiB, twice the 256 MB Infinity Cache), so every
      step streams its weights from HBM as a decoder walking many layers
      would.  Steps are captured in a HIP graph and replayed.  value = HBM
      GB/s of algorithmic bytes per step.
  ffn_4096: pack X (4096 x 4096 bf16) and run the alpha-scaled GEMM against
      packed W (11008 x 4096).  value = binary GOPS (2*M*N*K / s).
  chain_65536: pack X (65536 x 512 fp32), two sign->repack layers
      (512->256->128) and an alpha-scaled last layer (128->64), as one
      bnn_chain3 launch (the four separate launches are timed beside it).
      value = binary GOPS over the three layers.
  signw_gemv_4096 / signw_16384: real bf16 activations times packed sign
      weights (bnn_gemm_signw_bf16), batch-1 and 16384 x 1024 x 1024; both
      also appear in the default record under "signw".

"roofline" reports the dominant kernel of the step: its algorithmic bytes
(or binary ops) per launch divided by its average duration, measured here
with HIP events on the stream it runs on, against the MI355X peak that
bounds it.  "cpu_baseline" times the CPU oracle on a bounded sample of the
same workload on this host's cores.  "secondary" repeats the measurement
for the large-M GEMM (ffn_4096) so that both regimes appear in one record.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "binary GOPS (2·M·N·K bit-MAC/s) + batch-1 GEMV HBM GB/s vs peak"

HBM_PEAK_GBS = 8000.0
# VALU XOR + popcount issue peak, in binary ops (2 per bit-MAC) per second:
# 256 CU x 64 lanes/clk x 2.4 GHz = 3.93e13 32-bit lane-ops/s; one 64-bit
# word pair (64 bit-MACs = 128 binary ops) costs 4 lane-ops
# (2 v_xor_b32 + 2 v_bcnt_u32_b32).
VALU_LANE_OPS = 256 * 64 * 2.4e9
ALU_PEAK_BINARY_OPS = VALU_LANE_OPS / 4 * 128
# Dense FP4 MFMA peak of MI355X (published): 10.1 PFLOP/s.  The matrix-core
# kernel encodes +-1 as FP4, so one binary MAC is one FP4 MAC (2 ops).
MFMA_FP4_PEAK_OPS = 10.1e15
# Dense bf16 MFMA peak of MI355X (published): 2.5 PFLOP/s.
MFMA_BF16_PEAK = 2.5e15


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="gemv_4096",
                    choices=["gemv_4096", "ffn_4096", "chain_65536", "signw_gemv_4096",
                             "signw_16384"])
    ap.add_argument("--ring", type=int, default=256, help="distinct weight copies (gemv)")
    ap.add_argument("--rows", type=int, default=None,
                    help="gemv only: override N (weight rows) for the streaming-rate variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--eager", action="store_true",
                    help="gemv: launch the steps one by one instead of replaying a HIP graph "
                         "(for counter collection)")
    ap.add_argument("--calibrate-copy", type=int, default=None, metavar="MIB",
                    help="run 8 plain device copies of MIB MiB and exit (the reference kernel "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# GPU legs


def timed(fn, n, stream):
    """Run fn() n times between two HIP events on `stream` (after one untimed
    call); ms per call."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n


def kernel_sources_digest(names):
    """sha256 over the library sources a counter record was taken with."""
    import hashlib
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "packed_xor_popcount_amd",
                        "csrc")
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(root, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(profile_name, sources):
    """HBM bytes per launch from a committed counter summary under profiles/
    (FETCH_SIZE + WRITE_SIZE of the kernel, each scaled by the same counter's
    reading for a plain copy of known size).  None when the summary is
    missing or was taken with different kernel sources."""
    import re
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", profile_name)
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_sources_digest(sources):
        return None
    return float(t.group(1))


GEMV_SOURCES = ["gemv.hip", "sign_bits.h", "bnn_internal.h"]
MFMA_SOURCES = ["gemm_mfma.hip", "fp4_ops.h", "bnn_internal.h"]
CHAIN_SOURCES = ["chain.hip", "fp4_ops.h", "sign_bits.h", "bnn_internal.h"]
SIGNW_SOURCES = ["signw.hip", "bnn_internal.h"]


def ring_steps_ms(step, R, steps, warmup, eager):
    """ms per step of `steps` calls step(i % R): eager warmup, then R steps
    (one per ring entry) captured in a HIP graph and replayed, timed with HIP
    events on torch's current stream (the capture's launch stream).  With
    `eager` the steps are plain launches (for counter collection)."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for i in range(max(warmup, 1)):
        step(i % R)
    torch.cuda.synchronize()

    def graph_of(n):
        gr = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(dev)
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(gr, stream=s):
                for j in range(n):
                    step(j % R)
        torch.cuda.synchronize()
        return gr

    if eager:
        return timed(lambda: [step(i % R) for i in range(steps)], 1, stream) / steps
    full, rem = divmod(steps, R)
    g_full = graph_of(R) if full else None
    g_rem = graph_of(rem) if rem else None
    for gr in (g_full, g_rem):
        if gr is not None:
            gr.replay()
    torch.cuda.synchronize()

    def run_steps():
        for _ in range(full):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()

    return timed(run_steps, 1, stream) / steps


def gemv_leg(args, steps, warmup):
    import torch
    import packed_xor_popcount_amd as bnn
    import workloads
    dev = torch.device("cuda:0")
    d = workloads.make("gemv_4096")
    K = d["K"]
    kw = bnn.words(K)
    wp = bnn.pack_signs(d["w"].to(dev))
    alpha = d["alpha"].to(dev)
    N = wp.shape[0]
    if args.rows:  # streaming-rate variant: tile the same rows up to args.rows
        reps = -(-args.rows // N)
        wp = wp.repeat(reps, 1)[: args.rows].contiguous()
        alpha = alpha.repeat(reps)[: args.rows].contiguous()
        N = args.rows
    R = max(1, args.ring if not args.rows else max(1, min(args.ring, (1 << 30) // (N * kw * 8))))
    wring = wp.unsqueeze(0).repeat(R, 1, 1).contiguous()
    del wp
    g = workloads.generator(2002)
    xring = workloads.normal(g, R, 1, K).to(torch.bfloat16).to(dev)
    xring[0].copy_(d["x"].to(dev))
    y = torch.empty((1, N), dtype=torch.float32, device=dev)

    def step(j):
        # one launch: the bf16 row is sign-packed inside the GEMV kernel
        bnn.gemv_act(xring[j], wring[j], K, bnn.EPI_SCALED, alpha=alpha, out=y)

    ms_step = ring_steps_ms(step, R, steps, warmup, args.eager)
    # the step is one kernel: its average duration is the step time of
    # back-to-back graph launches (an upper bound: it includes launch gaps)
    ms_gemv = ms_step
    bytes_gemv = N * kw * 8 + K * 2 + N * 4 + N * 4           # Wp + x bf16 + alpha + y
    bytes_step = bytes_gemv
    gbs = bytes_step / (ms_step * 1e-3) / 1e9
    gops = 2.0 * N * K / (ms_step * 1e-3) / 1e9
    achieved = bytes_gemv / (ms_gemv * 1e-3) / 1e9
    return dict(
        value=gbs, unit="GB/s", ms_per_step=ms_step, binary_gops=gops,
        config={"workload": "gemv_4096" if not args.rows else f"gemv_4096_rows{N}", "M": 1,
                "K": K, "N": N, "x_dtype": "bf16", "w_dtype": "fp32 (packed offline)",
                "epilogue": "alpha-scaled fp32", "weight_ring": R,
                "bytes_per_step": bytes_step, "hip_graph": not args.eager},
        roofline={"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": achieved / HBM_PEAK_GBS,
                  "traffic": recorded_traffic("gemv_4096_traffic.md", GEMV_SOURCES)
                  if not args.rows else None,
                  "kernel": "gemv_act_kernel (bf16 activations packed in-kernel, alpha-scaled)",
                  "kernel_avg_us": ms_gemv * 1e3,
                  "algorithmic_bytes_per_launch": bytes_gemv},
        step_inputs=(d, N, K),
    )


def signw_gemv_leg(steps, warmup, ring=256, eager=False):
    """Batch-1 product of a real bf16 activation row with packed sign weights
    (bnn_gemm_signw_bf16, GEMV kernel) on the gemv_4096 inputs: x is used
    as is (not sign-projected), W is the same packed 4096 x 4096 matrix, with
    the same weight ring and HIP-graph replay as the binary GEMV step."""
    import torch
    import packed_xor_popcount_amd as bnn
    import workloads
    dev = torch.device("cuda:0")
    d = workloads.make("gemv_4096")
    K = d["K"]
    kw = bnn.words(K)
    wp = bnn.pack_signs(d["w"].to(dev))
    alpha = d["alpha"].to(dev)
    N = wp.shape[0]
    R = ring
    wring = wp.unsqueeze(0).repeat(R, 1, 1).contiguous()
    del wp
    g = workloads.generator(2003)
    xring = workloads.normal(g, R, 1, K).to(torch.bfloat16).to(dev)
    xring[0].copy_(d["x"].to(dev))
    y = torch.empty((1, N), dtype=torch.float32, device=dev)

    def step(j):
        bnn.gemm_signw_bf16(xring[j], wring[j], K, alpha, bnn.ALGO_GEMV, out=y)

    ms = ring_steps_ms(step, R, steps, warmup, eager)
    nbytes = N * kw * 8 + K * 2 + N * 4 + N * 4  # Wp + x bf16 + alpha + y
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "signw_gemv_4096", "value": ach, "unit": "GB/s", "ms_per_step": ms,
            "config": {"M": 1, "K": K, "N": N, "x_dtype": "bf16 (real-valued)",
                       "w_dtype": "packed signs", "epilogue": "alpha-scaled fp32",
                       "weight_ring": R, "hip_graph": not eager},
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS,
                         "traffic": recorded_traffic("signw_gemv_4096_traffic.md", SIGNW_SOURCES),
                         "kernel": "gemv_signw_kernel", "kernel_avg_us": ms * 1e3,
                         "algorithmic_bytes_per_launch": nbytes}}


def signw_cpu_baseline(workload, seconds):
    """The oracle's real-activation product (float64 sums) on a bounded
    sample of the same workload: whole batch-1 steps, or a few rows of the
    16384-row GEMM against every column."""
    import numpy as np
    import oracle
    import workloads
    d = workloads.make("gemv_4096" if workload == "signw_gemv_4096" else "signw_16384")
    K = d["K"]
    wp = oracle.pack(d["w"].numpy())
    N = wp.shape[0]
    rows = 1 if workload == "signw_gemv_4096" else 8
    xb = workloads.bf16_bits(d["x"][:rows])
    cores = os.cpu_count() or 1
    n, t0 = 0, time.perf_counter()
    while True:
        s = oracle.dot_signw_bf16(xb, wp, K, nthreads=cores)
        _ = s * d["alpha"].numpy().astype(np.float64)[None, :]
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    if rows == 1:
        nbytes = N * oracle.words(K) * 8 + K * 2 + 8 * N
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{n} full batch-1 steps, {dt * 1e3:.1f} ms each (one row: one thread)"}
    return {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TFLOP/s",
            "cores": min(cores, rows), "kind": "oracle",
            "sample": f"{n} x {rows} rows against all {N} columns, {dt * 1e3:.1f} ms each"}


def signw_gemm_leg(steps, warmup):
    """Real bf16 activations (16384 x 1024) times packed sign weights
    (1024 x 1024), alpha-scaled fp32 output: the largest packed-kernel shape
    of the binary_nn README's "Triton Kernel Benchmark" section."""
    import torch
    import packed_xor_popcount_amd as bnn
    import workloads
    dev = torch.device("cuda:0")
    d = workloads.make("signw_16384")
    M, K = d["x"].shape
    x = d["x"].to(dev)
    wp = bnn.pack_signs(d["w"].to(dev))
    alpha = d["alpha"].to(dev)
    N = wp.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        bnn.gemm_signw_bf16(x, wp, K, alpha, bnn.ALGO_AUTO, out=y)

    for _ in range(max(warmup, 1)):
        step()
    ms = timed(step, steps, stream)
    flops = 2.0 * M * N * K
    nbytes = M * K * 2 + N * bnn.words(K) * 8 + N * 4 + M * N * 4
    ach = flops / (ms * 1e-3)
    return {"workload": "signw_16384", "value": ach / 1e12, "unit": "TFLOP/s",
            "ms_per_step": ms,
            "config": {"M": M, "K": K, "N": N, "x_dtype": "bf16 (real-valued)",
                       "w_dtype": "packed signs", "epilogue": "alpha-scaled fp32"},
            "roofline": {"bound": "mfma", "achieved": ach / 1e12, "peak": MFMA_BF16_PEAK / 1e12,
                         "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK,
                         "traffic": recorded_traffic("signw_16384_traffic.md", SIGNW_SOURCES),
                         "kernel": "gemm_signw_kernel (bf16 MFMA)", "kernel_avg_us": ms * 1e3,
                         "algorithmic_flops_per_launch": flops,
                         "algorithmic_bytes_per_launch": nbytes,
                         "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def ffn_leg(steps, warmup):
    import torch
    import packed_xor_popcount_amd as bnn
    import workloads
    dev = torch.device("cuda:0")
    d = workloads.make("ffn_4096")
    K = d["K"]
    x = d["x"].to(dev)
    wp = bnn.pack_signs(d["w"].to(dev))
    alpha = d["alpha"].to(dev)
    M, N = x.shape[0], wp.shape[0]
    xp = torch.empty((M, bnn.words(K)), dtype=torch.int64, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        bnn.pack_signs(x, out=xp)
        bnn.gemm_ex(xp, wp, K, bnn.EPI_SCALED, bnn.ALGO_AUTO, alpha=alpha, out=y)

    def gemm(algo):
        return lambda: bnn.gemm_ex(xp, wp, K, bnn.EPI_SCALED, algo, alpha=alpha, out=y)

    for _ in range(max(warmup, 1)):
        step()
    ms_step = timed(step, steps, stream)
    ms_gemm = timed(gemm(bnn.ALGO_MFMA), steps, stream)       # what AUTO runs at this shape
    ms_valu = timed(gemm(bnn.ALGO_TILED), max(3, steps // 3), stream)  # the popcount ablation
    ops = 2.0 * M * N * K
    ach = ops / (ms_gemm * 1e-3)
    return dict(
        value=ops / (ms_step * 1e-3) / 1e9, unit="binary GOPS", ms_per_step=ms_step,
        config={"workload": "ffn_4096", "M": M, "K": K, "N": N, "x_dtype": "bf16",
                "w_dtype": "fp32 (packed offline)", "epilogue": "alpha-scaled fp32"},
        roofline={"bound": "mfma", "achieved": ach / 1e12, "peak": MFMA_FP4_PEAK_OPS / 1e12,
                  "unit": "T binary-ops/s (= FP4 TFLOP/s)", "frac": ach / MFMA_FP4_PEAK_OPS,
                  "traffic": recorded_traffic("ffn_4096_traffic.md", MFMA_SOURCES),
                  "kernel": "gemm_mfma_kernel (alpha-scaled)",
                  "kernel_avg_us": ms_gemm * 1e3, "algorithmic_ops_per_launch": ops,
                  "frac_of_valu_popcount_peak": ach / ALU_PEAK_BINARY_OPS},
        ablation={"valu_xor_popcount_us": ms_valu * 1e3, "mfma_fp4_us": ms_gemm * 1e3,
                  "valu_xor_popcount_frac_of_valu_peak": ops / (ms_valu * 1e-3) / ALU_PEAK_BINARY_OPS,
                  "speedup_mfma_over_valu": ms_valu / ms_gemm},
        step_inputs=(d, N, K),
    )


def thr_cpu_baseline(h0, w1, thr, flip, dims, rows=2048):
    """The oracle's threshold repack of chain layer 1 on its first `rows`
    packed input rows (the same operands the GPU leg times)."""
    import numpy as np
    import oracle
    xp = h0[:rows].cpu().numpy().view(np.uint64)
    wp = w1.cpu().numpy().view(np.uint64)
    t = thr.cpu().numpy()
    fl = np.unpackbits(flip.cpu().numpy().view(np.uint8), bitorder="little")[: dims[1]]
    cores = os.cpu_count() or 1
    n, t0 = 0, time.perf_counter()
    while n < 3 or time.perf_counter() - t0 < 1.0:
        oracle.sign_repack_thr(xp, wp, t, dims[0], fl, nthreads=cores)
        n += 1
    dt = (time.perf_counter() - t0) / n
    return {"value": 2.0 * rows * dims[0] * dims[1] / dt / 1e9, "unit": "binary GOPS",
            "cores": cores, "kind": "oracle",
            "sample": f"{n} x {rows} rows of layer 1, {dt * 1e3:.1f} ms each"}


def chain_leg(steps, warmup):
    import torch
    import packed_xor_popcount_amd as bnn
    import workloads
    dev = torch.device("cuda:0")
    d = workloads.make("chain_65536")
    dims = d["dims"]
    x = d["x"].to(dev)
    M = x.shape[0]
    wps = [bnn.pack_signs(w.to(dev)) for w in d["weights"]]
    alpha = d["alpha"].to(dev)
    h0 = torch.empty((M, bnn.words(dims[0])), dtype=torch.int64, device=dev)
    h1 = torch.empty((M, bnn.words(dims[1])), dtype=torch.int64, device=dev)
    h2 = torch.empty((M, bnn.words(dims[2])), dtype=torch.int64, device=dev)
    y = torch.empty((M, dims[3]), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        bnn.pack_signs(x, out=h0)
        bnn.gemm_sign_repack(h0, wps[0], dims[0], out=h1)
        bnn.gemm_sign_repack(h1, wps[1], dims[1], out=h2)
        bnn.gemm_u64_scaled(h2, wps[2], alpha, dims[2], out=y)

    def fused():
        # the same step in one launch: pack, two repack layers and the scaled
        # layer with the packed hidden rows kept on chip (bit-identical)
        bnn.chain3(x, wps[0], wps[1], wps[2], alpha, out=y)

    # layer 1 with a folded BatchNorm (per-channel threshold + flip mask)
    # against the plain sign -> repack of the same layer
    g = workloads.generator(3003)
    thr = (workloads.normal(g, dims[1]) * 8).round().to(torch.int32).to(dev)
    flip = bnn.flip_words((workloads.normal(g, dims[1]) < 0).to(torch.int32).to(dev))

    def layer1():
        bnn.gemm_sign_repack(h0, wps[0], dims[0], out=h1)

    def layer1_thr():
        bnn.gemm_sign_repack_thr(h0, wps[0], thr, dims[0], flip, out=h1)

    for _ in range(max(warmup, 1)):
        step()
        fused()
    ms_sep = timed(step, steps, stream)
    ms_step = timed(fused, steps, stream)
    ms_l1 = timed(layer1, steps, stream)
    ms_l1_thr = timed(layer1_thr, steps, stream)
    ops = sum(2.0 * M * dims[i] * dims[i + 1] for i in range(3))
    # HBM bytes of the fused launch: the fp32 input, the fp32 output, the
    # packed weights and the scales
    nbytes = (M * dims[0] * 4 + M * dims[3] * 4 + sum(w.numel() * 8 for w in wps)
              + dims[3] * 4)
    ach = nbytes / (ms_step * 1e-3) / 1e9
    return dict(
        value=ops / (ms_step * 1e-3) / 1e9, unit="binary GOPS", ms_per_step=ms_step,
        config={"workload": "chain_65536", "M": M, "dims": list(dims), "x_dtype": "fp32",
                "hidden": "sign->repack u64", "epilogue": "alpha-scaled fp32",
                "launch": "bnn_chain3 (fused)"},
        roofline={"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": ach / HBM_PEAK_GBS,
                  "traffic": recorded_traffic("chain_65536_traffic.md", CHAIN_SOURCES),
                  "kernel": "chain3_kernel (pack + 3 layers, one launch)",
                  "kernel_avg_us": ms_step * 1e3, "algorithmic_bytes_per_launch": nbytes,
                  "mfma_frac": ops / (ms_step * 1e-3) / MFMA_FP4_PEAK_OPS},
        unfused={"us_per_step": ms_sep * 1e3, "launches": 4,
                 "value": ops / (ms_sep * 1e-3) / 1e9},
        threshold_repack={"layer": "512 -> 256 at M=65536 (gemm_mfma_kernel)",
                          "plain_us": ms_l1 * 1e3, "threshold_flip_us": ms_l1_thr * 1e3,
                          "binary_gops": 2.0 * M * dims[0] * dims[1] / (ms_l1_thr * 1e-3) / 1e9,
                          "cpu_baseline": thr_cpu_baseline(h0, wps[0], thr, flip, dims)},
        step_inputs=(d, None, None),
    )


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of the workload


def cpu_baseline(workload, step_inputs, seconds):
    import numpy as np
    import oracle
    import workloads
    d, N, K = step_inputs
    if workload == "gemv_4096":
        wp = oracle.pack(d["w"].numpy())   # weights are packed offline, as on the GPU
        alpha = d["alpha"].numpy()
        xb = workloads.bf16_bits(d["x"])
        kw = oracle.words(K)
        bytes_step = N * kw * 8 + K * 2 + N * 8   # as the GPU step: Wp + x bf16 + alpha + y
        n, t0 = 0, time.perf_counter()
        while True:
            xp = oracle.pack(xb)
            oracle.gemm_scaled(xp, wp, alpha, K)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = (time.perf_counter() - t0) / n
        return {"value": bytes_step / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{n} full gemv_4096 steps (pack x + scaled GEMV), {dt * 1e3:.1f} ms/step;"
                          " the oracle splits rows over threads, and M=1 gives one thread"}
    if workload == "ffn_4096":
        rows = 8
        xb = workloads.bf16_bits(d["x"][:rows])
        wp = oracle.pack(d["w"].numpy())
        alpha = d["alpha"].numpy()
        cores = os.cpu_count() or 1
        n, t0 = 0, time.perf_counter()
        while True:
            xp = oracle.pack(xb)
            oracle.gemm_scaled(xp, wp, alpha, K, nthreads=cores)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = (time.perf_counter() - t0) / n
        return {"value": 2.0 * rows * N * K / dt / 1e9, "unit": "binary GOPS",
                "cores": min(cores, rows), "kind": "oracle",
                "sample": f"{n} x {rows} rows of ffn_4096 (all 11008 columns), {dt:.2f} s each"}
    # chain
    rows = 2048
    x = d["x"].numpy()[:rows]
    ws = [w.numpy() for w in d["weights"]]
    cores = os.cpu_count() or 1
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.chain(x, ws, d["alpha"].numpy(), nthreads=cores)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    dims = d["dims"]
    ops = sum(2.0 * rows * dims[i] * dims[i + 1] for i in range(3))
    return {"value": ops / dt / 1e9, "unit": "binary GOPS", "cores": cores, "kind": "oracle",
            "sample": f"{n} x {rows}-row chain passes, {dt:.2f} s each"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this implementation has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a visible MI355X GPU", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import packed_xor_popcount_amd as bnn
    bnn.library()  # fail loudly if the HIP library is missing
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.calibrate_copy} MiB x 8")
        return

    defaults = {"gemv_4096": (1024, 64), "ffn_4096": (20, 3), "chain_65536": (50, 5),
                "signw_gemv_4096": (1024, 64), "signw_16384": (50, 5)}
    steps = args.steps if args.steps is not None else defaults[args.workload][0]
    warmup = args.warmup if args.warmup is not None else defaults[args.workload][1]
    log(f"[bench] workload={args.workload} steps={steps} warmup={warmup}")
    if args.workload == "gemv_4096":
        res = gemv_leg(args, steps, warmup)
    elif args.workload == "ffn_4096":
        res = ffn_leg(steps, warmup)
    elif args.workload == "chain_65536":
        res = chain_leg(steps, warmup)
    else:
        leg = (signw_gemv_leg(steps, warmup, args.ring, args.eager)
               if args.workload == "signw_gemv_4096" else signw_gemm_leg(steps, warmup))
        res = dict(leg, config=dict(leg["config"], workload=leg["workload"]), step_inputs=None)
    log(f"[bench] {args.workload}: {res['value']:.1f} {res['unit']}, "
        f"{res['ms_per_step'] * 1e3:.2f} us/step")

    out = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u64",
        "data": "synthetic (seeded, see workloads.py)", "config": res["config"],
        "roofline": res["roofline"],
    }
    if "binary_gops" in res:
        out["binary_gops"] = res["binary_gops"]
    if "ablation" in res:
        out["ablation"] = res["ablation"]
    if "unfused" in res:
        out["unfused"] = res["unfused"]
    if "threshold_repack" in res:
        out["threshold_repack"] = res["threshold_repack"]
    if args.workload == "gemv_4096" and not args.no_secondary and not args.rows:
        sec = ffn_leg(10, 2)
        log(f"[bench] secondary ffn_4096: {sec['value']:.1f} binary GOPS")
        out["secondary"] = {"workload": "ffn_4096", "value": sec["value"], "unit": sec["unit"],
                            "ms_per_step": sec["ms_per_step"], "roofline": sec["roofline"],
                            "ablation": sec["ablation"]}
    if args.workload == "gemv_4096" and not args.no_secondary and not args.rows:
        # the real-activation product (packed sign weights), both regimes
        out["signw"] = []
        for leg in (signw_gemv_leg(1024, 64), signw_gemm_leg(20, 3)):
            log(f"[bench] {leg['workload']}: {leg['value']:.1f} {leg['unit']}, "
                f"{leg['ms_per_step'] * 1e3:.2f} us/step")
            rec = {k: leg[k] for k in ("workload", "value", "unit", "ms_per_step", "config",
                                       "roofline")}
            if not args.no_cpu_baseline:
                rec["cpu_baseline"] = signw_cpu_baseline(leg["workload"], 3.0)
            out["signw"].append(rec)
    if not args.no_cpu_baseline and args.workload.startswith("signw"):
        log("[bench] timing the CPU oracle ...")
        out["cpu_baseline"] = signw_cpu_baseline(args.workload, args.cpu_seconds)
    if not args.no_cpu_baseline and res["step_inputs"] is not None:
        log("[bench] timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(args.workload, res["step_inputs"], args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
