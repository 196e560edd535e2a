#!/usr/bin/env python3
"""Benchmark of the packed binary (XOR + popcount) hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Prints ONE JSON line.  A step is one pass of the hot path over one batch of
synthetic input, inputs already resident in HBM.

The headline line (default workload gemv_4096) is the batch-1 binary GEMV,
M = 1, K = N = 4096: one launch of bnn_gemv_act sign-packs the bf16
activation row inside the kernel and runs the alpha-scaled fp32 product
against a packed 4096 x 4096 weight matrix (2 MiB).  The weights are cold in
every timed step: step i reads weight copy i mod R of a ring of R = 384
distinct copies (768 MiB, three times the 256 MB Infinity Cache), and the
copies a timed step reads were last touched before 383 other copies (766 MiB)
were read (see ring_plan).  Exactly K steps are captured in a
HIP graph and replayed between two HIP events.  value = algorithmic HBM
bytes per step / step time.

The same JSON line carries, as nested records, every other measurement of
the path (each with its own roofline and CPU-oracle baseline):

  streaming      the same kernel streaming 512 MiB of packed weights per
                 launch (N = 1 048 576 rows), cold: its HBM rate.
  named_batch1   the named entry points at batch 1: bnn_gemm_u64_scaled on a
                 prepacked activation row (one launch) and the pack_signs +
                 bnn_gemm_u64_scaled sequence (two launches).
  secondary      ffn_4096: pack X (4096 x 4096 bf16) and the alpha-scaled
                 GEMM against packed W (11008 x 4096); binary GOPS; the VALU
                 XOR + popcount kernel timed beside it (ablation).
  chain          chain_65536: pack + 512 -> 256 -> 128 (sign -> repack) ->
                 64 (alpha-scaled), one fused launch, the four separate
                 launches, and the threshold repack of layer 1.
  signw          real bf16 activations times packed sign weights, batch-1
                 and 16384 x 1024 x 1024.
  small          gemv_small and edge_1000 (latency-bound), with single-thread
                 oracle times.
  calibration    the rates this GPU sustains on register-only probes (VALU
                 xor + popcount pairs, FP4 MFMA on fixed and on changing +-1
                 operands) and a streaming HBM read, with the shader clock
                 measured during each probe, and the cost of one launch of
                 the batch-1 grid with no work in it; every roofline
                 carries its fraction of the matching calibrated rate next
                 to its fraction of the published peak.

"roofline" reports the dominant kernel of a step: algorithmic bytes (or
binary ops) per launch divided by its average launch duration, measured
here with HIP events on the stream it is launched on, against the MI355X
peak that bounds it.  "cpu_baseline" times the CPU oracle on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
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
# kernels encode +-1 as FP4, so one binary MAC is one FP4 MAC (2 ops).
MFMA_FP4_PEAK_OPS = 10.1e15
# Dense bf16 MFMA peak of MI355X (published): 2.5 PFLOP/s.
MFMA_BF16_PEAK = 2.5e15
MALL_BYTES = 256 * 2 ** 20   # Infinity Cache
GEMV_RING = 384              # weight copies of the batch-1 ring (768 MiB)
STREAM_ROWS = 1 << 20        # streaming variant: 512 MiB of packed weights


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="gemv_4096",
                    choices=["gemv_4096", "gemv_stream", "named_gemv_4096", "ffn_4096",
                             "chain_65536", "signw_gemv_4096", "signw_16384", "small",
                             "calibrate"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-nested", action="store_true",
                    help="headline line only (no nested records, no calibration)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--eager", action="store_true",
                    help="ring workloads: launch the steps one by one instead of replaying a "
                         "HIP graph (for counter collection)")
    ap.add_argument("--calibrate-copy", type=int, default=None, metavar="MIB",
                    help="run 8 plain device copies of MIB MiB and exit (the reference kernel "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args(argv)


# ---------------------------------------------------------------------------
# Cold-weight ring protocol (host logic, tested without a GPU)


def ring_plan(R: int, steps: int, warmup: int):
    """Order in which ring entries are read around the timed region.

    Returns a list of (phase, entries) in execution order:
      ("warm", ...)    eager warm-up steps, on entries the timed region does
                       not read when steps + warmup <= R;
      ("graph", ...)   one replay of the timed graph (graph warm-up);
      ("evict", ...)   eager steps over the entries after the last one the
                       graph replay read (when steps is not a multiple of R),
                       so that the timed replay starts R - 1 entries after
                       the previous read of its first entry;
      ("timed", ...)   the timed replay: step i reads entry i mod R.
    With steps >= R every entry is timed, and between two reads of an entry
    the other R - 1 entries are read."""
    timed = [i % R for i in range(steps)]
    # entries after the last one the timed region reads (its first pass when
    # steps < R, its remainder pass otherwise)
    rest = list(range(steps % R, R)) if steps % R else []
    if steps < R:
        warm = [rest[(len(rest) - 1 - i) % len(rest)] for i in range(warmup)]
    else:
        warm = [(R - 1 - i) % R for i in range(warmup)]
    plan = [("warm", warm), ("graph", timed)]
    if rest:
        plan.append(("evict", rest))
    plan.append(("timed", timed))
    return plan


def cold_gap_entries(plan) -> int:
    """Smallest number of reads of OTHER ring entries between a timed read
    and the previous read of the same entry (the timed reads included, so a
    ring shorter than the step count is covered too)."""
    seq = [e for _, ents in plan for e in ents]
    t0 = len(seq) - len(plan[-1][1])
    last = {}
    gap = None
    for i, e in enumerate(seq):
        if i >= t0 and e in last:
            g = i - last[e] - 1
            gap = g if gap is None else min(gap, g)
        last[e] = i
    return gap if gap is not None else len(seq)


def ring_steps_ms(step, R, steps, warmup, eager=False):
    """ms per step of `steps` calls step(i % R), following ring_plan: the
    timed steps are captured in a HIP graph (R-step graph replayed, plus a
    remainder graph) and timed with HIP events on torch's current stream
    (the capture's launch stream); with `eager` they are plain launches (for
    counter collection).  Returns (ms per step, protocol record)."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    plan = ring_plan(R, steps, warmup)
    phases = dict(plan)
    for j in phases["warm"]:
        step(j)
    torch.cuda.synchronize()

    def graph_of(entries):
        gr = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(dev)
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(gr, stream=s):
                for j in entries:
                    step(j)
        torch.cuda.synchronize()
        return gr

    full, rem = divmod(steps, R)
    if eager:
        def run_timed():
            for j in phases["timed"]:
                step(j)
    else:
        g_full = graph_of(list(range(R))) if full else None
        g_rem = graph_of(list(range(rem))) if rem else None

        def run_timed():
            for _ in range(full):
                g_full.replay()
            if g_rem is not None:
                g_rem.replay()
    run_timed()  # the "graph" phase: first replay of the timed graph(s)
    for j in phases.get("evict", []):
        step(j)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    run_timed()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    proto = {"ring_entries": R, "distinct_timed_entries": min(steps, R),
             "cold_gap_entries": cold_gap_entries(plan), "hip_graph": not eager}
    if not eager and steps < R:
        # Each graph replay carries a fixed cost outside its kernels (about
        # 11 us on this platform), which a short replay spreads over few
        # steps.  For reference, the same steps over the whole ring in one
        # replay, starting after the entries just timed (so that these are
        # read last, after the R - steps others): the per-step time of a
        # long run.
        order = [(steps + i) % R for i in range(R)]
        g_all = graph_of(order)
        g_all.replay()  # untimed first replay: between two reads of an entry, R - 1 others
        torch.cuda.synchronize()
        start.record(stream)
        g_all.replay()
        end.record(stream)
        torch.cuda.synchronize()
        proto["ring_pass_us_per_step"] = start.elapsed_time(end) / R * 1e3
    return ms, proto


def roof_with_ring_pass(roof, proto):
    """Move the long-run per-step time of a short ring run from the protocol
    record into the roofline record, beside the kernel's average duration."""
    v = proto.pop("ring_pass_us_per_step", None)
    if v is not None:
        roof = dict(roof, ring_pass_us_per_step=v)
    return roof


# ---------------------------------------------------------------------------
# Timing helpers


def event_split(fns, n, stream):
    """Run the callables `fns` in order, n times, with a HIP event on `stream`
    before the first and after each; returns (per-callable lists of ms, list
    of whole-step ms)."""
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(n)]
    for i in range(n):
        evs[i][0].record(stream)
        for j, f in enumerate(fns):
            f()
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    per = [[evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(n)] for j in range(len(fns))]
    whole = [evs[i][0].elapsed_time(evs[i][-1]) for i in range(n)]
    return per, whole


def graph_ms(fn, n, warm=3):
    """ms per call of fn() captured n times in one HIP graph (latency-bound
    work: no launch gap from Python between the calls)."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(dev)
    s.wait_stream(stream)
    with torch.cuda.stream(s):
        with torch.cuda.graph(gr, stream=s):
            for _ in range(n):
                fn()
    torch.cuda.synchronize()
    gr.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    gr.replay()
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


def with_calibration(roof, calib, kind):
    """Add the calibrated peak of `kind` ("hbm", "mfma_fp4", "valu") to a
    roofline record: its fraction and the shader clock of the probe."""
    if not calib or kind not in calib:
        return roof
    c = calib[kind]
    roof = dict(roof)
    roof["calibrated_peak"] = c["rate"]
    roof["calibrated_frac"] = roof["achieved"] / c["rate"]
    if c.get("sclk_mhz"):
        roof["sclk_mhz"] = c["sclk_mhz"]
    return roof


# ---------------------------------------------------------------------------
# Calibration probes


def calibrate():
    """Rates of register-only VALU xor + popcount and FP4 MFMA loops and of a
    1 GiB streaming read, each the median of 3 runs timed with HIP events,
    with the shader clock from the probes' cycle and wall counters."""
    import torch
    from packed_xor_popcount_amd import calib as cal
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    wall_hz = cal.wallclock_hz()

    def run(fn, n=3):
        fn()
        torch.cuda.synchronize()
        times, clocks = [], []
        for _ in range(n):
            (ms,), _ = event_split([fn], 1, stream)
            rec = run.last.cpu()
            times.append(ms[0])
            dc = (rec[:, 1] - rec[:, 0]).double()
            dw = (rec[:, 3] - rec[:, 2]).double()
            ok = dw > 0
            if wall_hz and ok.any():
                clocks.append(float((dc[ok] / dw[ok]).median()) * wall_hz / 1e6)
        return statistics.median(times), (statistics.median(clocks) if clocks else None)

    out = {"wallclock_hz": wall_hz}
    vb, vi = 256 * 8, 4096

    def v():
        run.last = cal.valu(vb, vi)
    ms, mhz = run(v)
    lane_ops = vb * 256 * 64 * vi
    rate = lane_ops / (ms * 1e-3)
    out["valu"] = {"rate": rate / 4 * 128 / 1e12, "unit": "T binary-ops/s (xor+popcount)",
                   "lane_ops_per_s": rate, "frac_of_nominal": rate / VALU_LANE_OPS,
                   "sclk_mhz": mhz, "probe": f"{vb} blocks x 256 threads x {vi} x 64 lane-ops"}
    mb, mi = 256 * 4, 16384

    def m():
        run.last = cal.mfma_fp4(mb, mi)
    ms, mhz = run(m)
    flops = mb * 4 * 4 * mi * 131072
    rate = flops / (ms * 1e-3)
    out["mfma_fp4"] = {"rate": rate / 1e12, "unit": "TFLOP/s (FP4)",
                       "frac_of_nominal": rate / MFMA_FP4_PEAK_OPS, "sclk_mhz": mhz,
                       "probe": f"{mb} blocks x 4 waves x {mi} x 4 MFMA 32x32x64 FP4"}

    def mp():
        run.last = cal.mfma_fp4_pm1(mb, mi)
    ms, mhz = run(mp)
    rate = flops / (ms * 1e-3)
    out["mfma_fp4_pm1"] = {"rate": rate / 1e12, "unit": "TFLOP/s (FP4)",
                           "frac_of_nominal": rate / MFMA_FP4_PEAK_OPS, "sclk_mhz": mhz,
                           "probe": f"{mb} blocks x 4 waves x {mi} x 4 MFMA 32x32x64 FP4 on "
                                    "pseudo-random +-1 operands, another pair each MFMA"}
    # Launch floor: back-to-back graph replays of a kernel that does almost
    # nothing (the VALU probe with one iteration) on the batch-1 GEMV's grid
    # of 512 blocks x 256 threads.
    import ctypes
    lib = cal.library()
    rec = torch.zeros(4 * 512 + 1, dtype=torch.int64, device=dev)

    def noop():
        st = lib.bnn_calib_valu(ctypes.c_void_p(rec.data_ptr()), 512, 1,
                                ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        if st != 0:
            raise RuntimeError(f"bnn_calib_valu: status {st}")
    out["launch_floor"] = {"us": graph_ms(noop, 1024) * 1e3,
                           "probe": "HIP graph of 1024 launches of 512 blocks x 256 threads, "
                                    "64 register-only lane-ops per thread"}
    buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
    best = None
    for rb in (1024, 2048, 4096, 8192):   # the best launch shape is the calibrated rate

        def r():
            run.last = cal.read(buf, rb)
        ms, mhz = run(r)
        if best is None or ms < best[0]:
            best = (ms, mhz, rb)
    ms, mhz, rb = best
    out["hbm"] = {"rate": buf.numel() / (ms * 1e-3) / 1e9, "unit": "GB/s",
                  "frac_of_nominal": buf.numel() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "sclk_mhz": mhz,
                  "probe": f"1 GiB read once, 16-byte nt loads, a contiguous 32 KiB per block "
                           f"step; best of 1024-8192 blocks ({rb})"}
    del buf
    return out


# ---------------------------------------------------------------------------
# GPU legs


def gemv_leg(steps, warmup, calib=None, rows=None, eager=False):
    """Batch-1 step (bnn_gemv_act, bf16 x packed in-kernel, alpha-scaled)
    over a cold weight ring; rows > 4096 tiles the weight rows up to `rows`
    (the streaming variant)."""
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
    if rows:  # streaming-rate variant: tile the same rows up to `rows`
        reps = -(-rows // N)
        wp = wp.repeat(reps, 1)[:rows].contiguous()
        alpha = alpha.repeat(reps)[:rows].contiguous()
        N = rows
    w_bytes = N * kw * 8
    R = GEMV_RING if not rows else max(2, -(-3 * MALL_BYTES // w_bytes))
    wring = wp.unsqueeze(0).repeat(R, 1, 1).contiguous()
    del wp
    g = workloads.generator(2002)
    xring = workloads.normal(g, R, 1, K).to(torch.bfloat16).to(dev)
    xring[0].copy_(d["x"].to(dev))
    y = torch.empty((1, N), dtype=torch.float32, device=dev)

    def step(j):
        # one launch: the bf16 row is sign-packed inside the GEMV kernel
        bnn.gemv_act(xring[j], wring[j], K, bnn.EPI_SCALED, alpha=alpha, out=y)

    ms, proto = ring_steps_ms(step, R, steps, warmup, eager)
    del wring
    nbytes = w_bytes + K * 2 + N * 4 + N * 4           # Wp + x bf16 + alpha + y
    gbs = nbytes / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": recorded_traffic("gemv_4096_traffic.md" if not rows
                                        else "gemv_stream_traffic.md", GEMV_SOURCES),
            "kernel": "gemv_act_kernel (bf16 activations packed in-kernel, alpha-scaled)",
            "kernel_avg_us": ms * 1e3, "algorithmic_bytes_per_launch": nbytes,
            "note": "a step is one launch: the kernel's average duration is the step time of "
                    "back-to-back graph replays (an upper bound: it includes launch gaps)"}
    roof = roof_with_ring_pass(roof, proto)
    if calib and "launch_floor" in calib and not rows:
        # what a launch of this grid costs with no work in it (same replay method)
        roof["launch_floor_us"] = calib["launch_floor"]["us"]
    return dict(
        value=gbs, unit="GB/s", ms_per_step=ms, binary_gops=2.0 * N * K / (ms * 1e-3) / 1e9,
        config={"workload": "gemv_4096" if not rows else f"gemv_4096_stream_rows{N}", "M": 1,
                "K": K, "N": N, "x_dtype": "bf16", "w_dtype": "fp32 (packed offline)",
                "epilogue": "alpha-scaled fp32", "bytes_per_step": nbytes, **proto},
        roofline=with_calibration(roof, calib, "hbm"),
        step_inputs=(d, N, K),
    )


def named_gemv_leg(steps, warmup, calib=None):
    """The named C-ABI entry points at batch 1 on the gemv_4096 inputs:
    bnn_gemm_u64_scaled on a prepacked activation row (one launch), and the
    pack_signs + bnn_gemm_u64_scaled sequence (two launches), each over the
    cold weight ring."""
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
    R = GEMV_RING
    wring = wp.unsqueeze(0).repeat(R, 1, 1).contiguous()
    del wp
    g = workloads.generator(2004)
    xring = workloads.normal(g, R, 1, K).to(torch.bfloat16).to(dev)
    xring[0].copy_(d["x"].to(dev))
    xpring = torch.stack([bnn.pack_signs(xring[j]) for j in range(R)])
    y = torch.empty((1, N), dtype=torch.float32, device=dev)
    xp1 = torch.empty((1, kw), dtype=torch.int64, device=dev)

    def gemv_only(j):
        bnn.gemm_u64_scaled(xpring[j], wring[j], alpha, K, out=y)

    def pack_then_gemv(j):
        bnn.pack_signs(xring[j], out=xp1)
        bnn.gemm_u64_scaled(xp1, wring[j], alpha, K, out=y)

    ms1, proto = ring_steps_ms(gemv_only, R, steps, warmup)
    ms2, proto2 = ring_steps_ms(pack_then_gemv, R, steps, warmup)
    del wring
    nbytes = N * kw * 8 + kw * 8 + N * 4 + N * 4   # Wp + xp + alpha + y
    gbs = nbytes / (ms1 * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": recorded_traffic("named_gemv_4096_traffic.md", GEMV_SOURCES),
            "kernel": "gemv_act_kernel (packed activations, alpha-scaled), via "
                      "bnn_gemm_u64_scaled",
            "kernel_avg_us": ms1 * 1e3, "algorithmic_bytes_per_launch": nbytes}
    roof = roof_with_ring_pass(roof, proto)
    return {"workload": "named_gemv_4096", "value": gbs, "unit": "GB/s", "ms_per_step": ms1,
            "config": {"M": 1, "K": K, "N": N, "x": "prepacked u64 row",
                       "call": "bnn_gemm_u64_scaled", **proto},
            "roofline": with_calibration(roof, calib, "hbm"),
            "pack_then_gemm": {"calls": "bnn_pack_signs + bnn_gemm_u64_scaled (2 launches)",
                               "us_per_step": ms2 * 1e3,
                               "value": (nbytes + K * 2) / (ms2 * 1e-3) / 1e9, "unit": "GB/s",
                               **({"ring_pass_us_per_step": proto2["ring_pass_us_per_step"]}
                                  if "ring_pass_us_per_step" in proto2 else {})}}


def signw_gemv_leg(steps, warmup, calib=None, eager=False):
    """Batch-1 product of a real bf16 activation row with packed sign weights
    (bnn_gemm_signw_bf16, GEMV kernel) on the gemv_4096 inputs: x is used
    as is (not sign-projected), W is the same packed 4096 x 4096 matrix, with
    the same cold weight ring and HIP-graph replay as the binary GEMV step."""
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
    R = GEMV_RING
    wring = wp.unsqueeze(0).repeat(R, 1, 1).contiguous()
    del wp
    g = workloads.generator(2003)
    xring = workloads.normal(g, R, 1, K).to(torch.bfloat16).to(dev)
    xring[0].copy_(d["x"].to(dev))
    y = torch.empty((1, N), dtype=torch.float32, device=dev)

    def step(j):
        bnn.gemm_signw_bf16(xring[j], wring[j], K, alpha, bnn.ALGO_GEMV, out=y)

    ms, proto = ring_steps_ms(step, R, steps, warmup, eager)
    del wring
    nbytes = N * kw * 8 + K * 2 + N * 4 + N * 4  # Wp + x bf16 + alpha + y
    ach = nbytes / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS,
            "traffic": recorded_traffic("signw_gemv_4096_traffic.md", SIGNW_SOURCES),
            "kernel": "gemv_signw_kernel", "kernel_avg_us": ms * 1e3,
            "algorithmic_bytes_per_launch": nbytes}
    roof = roof_with_ring_pass(roof, proto)
    return {"workload": "signw_gemv_4096", "value": ach, "unit": "GB/s", "ms_per_step": ms,
            "config": {"M": 1, "K": K, "N": N, "x_dtype": "bf16 (real-valued)",
                       "w_dtype": "packed signs", "epilogue": "alpha-scaled fp32", **proto},
            "roofline": with_calibration(roof, calib, "hbm")}


def signw_gemm_leg(n, calib=None):
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

    for _ in range(3):
        step()
    (t,), _ = event_split([step], n, stream)
    ms = statistics.fmean(t)
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
                         "kernel_median_us": statistics.median(t) * 1e3,
                         "algorithmic_flops_per_launch": flops,
                         "algorithmic_bytes_per_launch": nbytes,
                         "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def ffn_leg(n, calib=None):
    """ffn_4096 step = pack X (bf16) + alpha-scaled GEMM (AUTO: the FP4 MFMA
    kernel).  Each step is bracketed by HIP events before the pack, between
    the two launches and after the GEMM, so the GEMM's average duration comes
    from the same launches as the step time.  The VALU XOR + popcount kernel
    is timed interleaved with the MFMA kernel (ablation)."""
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

    def pack():
        bnn.pack_signs(x, out=xp)

    def gemm():
        bnn.gemm_u64_scaled(xp, wp, alpha, K, out=y)

    def gemm_valu():
        bnn.gemm_ex(xp, wp, K, bnn.EPI_SCALED, bnn.ALGO_TILED, alpha=alpha, out=y)

    for _ in range(3):
        pack()
        gemm()
    (t_pack, t_gemm), t_step = event_split([pack, gemm], n, stream)
    gemm_valu()
    (t_mfma, t_valu), _ = event_split([gemm, gemm_valu], max(3, n // 4), stream)
    ops = 2.0 * M * N * K
    ms_step, ms_gemm = statistics.fmean(t_step), statistics.fmean(t_gemm)
    ach = ops / (ms_gemm * 1e-3)
    ms_valu, ms_mfma2 = statistics.fmean(t_valu), statistics.fmean(t_mfma)
    roof = {"bound": "mfma", "achieved": ach / 1e12, "peak": MFMA_FP4_PEAK_OPS / 1e12,
            "unit": "T binary-ops/s (= FP4 TFLOP/s)", "frac": ach / MFMA_FP4_PEAK_OPS,
            "traffic": recorded_traffic("ffn_4096_traffic.md", MFMA_SOURCES),
            "kernel": "gemm_mfma_kernel (alpha-scaled)",
            "kernel_avg_us": ms_gemm * 1e3, "kernel_median_us": statistics.median(t_gemm) * 1e3,
            "launches_timed": n, "algorithmic_ops_per_launch": ops,
            "frac_of_valu_popcount_peak": ach / ALU_PEAK_BINARY_OPS}
    roof = with_calibration(roof, calib, "mfma_fp4")
    if calib and "mfma_fp4_pm1" in calib:
        # the matrix cores' rate on +-1 operands that change every MFMA (the
        # data this product feeds them)
        roof["calibrated_pm1_peak"] = calib["mfma_fp4_pm1"]["rate"]
        roof["calibrated_pm1_frac"] = roof["achieved"] / calib["mfma_fp4_pm1"]["rate"]
    valu_rate = ops / (ms_valu * 1e-3)
    abl = {"valu_xor_popcount_us": ms_valu * 1e3, "mfma_fp4_us": ms_mfma2 * 1e3,
           "valu_xor_popcount_frac_of_valu_peak": valu_rate / ALU_PEAK_BINARY_OPS,
           "speedup_mfma_over_valu": ms_valu / ms_mfma2, "launches_timed": len(t_valu)}
    if calib and "valu" in calib:
        abl["valu_xor_popcount_calibrated_frac"] = valu_rate / 1e12 / calib["valu"]["rate"]
    return dict(
        value=ops / (ms_step * 1e-3) / 1e9, unit="binary GOPS", ms_per_step=ms_step,
        config={"workload": "ffn_4096", "M": M, "K": K, "N": N, "x_dtype": "bf16",
                "w_dtype": "fp32 (packed offline)", "epilogue": "alpha-scaled fp32",
                "pack_us": statistics.fmean(t_pack) * 1e3},
        roofline=roof, ablation=abl, step_inputs=(d, N, K),
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


def chain_leg(n, calib=None, cpu=True):
    """chain_65536: the fused launch (bnn_chain3) is the step; the four
    separate launches and the threshold repack of layer 1 are timed beside
    it, interleaved."""
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

    def separate():
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

    for _ in range(3):
        separate()
        fused()
    (t_fused, t_sep, t_l1, t_l1t), _ = event_split([fused, separate, layer1, layer1_thr], n,
                                                    stream)
    ms_step = statistics.fmean(t_fused)
    ms_sep = statistics.fmean(t_sep)
    ops = sum(2.0 * M * dims[i] * dims[i + 1] for i in range(3))
    # HBM bytes of the fused launch: the fp32 input, the fp32 output, the
    # packed weights and the scales
    nbytes = (M * dims[0] * 4 + M * dims[3] * 4 + sum(w.numel() * 8 for w in wps)
              + dims[3] * 4)
    ach = nbytes / (ms_step * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS,
            "traffic": recorded_traffic("chain_65536_traffic.md", CHAIN_SOURCES),
            "kernel": "chain3_kernel (pack + 3 layers, one launch)",
            "kernel_avg_us": ms_step * 1e3, "kernel_median_us": statistics.median(t_fused) * 1e3,
            "launches_timed": n, "algorithmic_bytes_per_launch": nbytes,
            "mfma_frac": ops / (ms_step * 1e-3) / MFMA_FP4_PEAK_OPS}
    res = dict(
        value=ops / (ms_step * 1e-3) / 1e9, unit="binary GOPS", ms_per_step=ms_step,
        config={"workload": "chain_65536", "M": M, "dims": list(dims), "x_dtype": "fp32",
                "hidden": "sign->repack u64", "epilogue": "alpha-scaled fp32",
                "launch": "bnn_chain3 (fused)"},
        roofline=with_calibration(roof, calib, "hbm"),
        unfused={"us_per_step": ms_sep * 1e3, "launches": 4,
                 "value": ops / (ms_sep * 1e-3) / 1e9, "unit": "binary GOPS",
                 "hbm_gbs_of_fused_bytes": nbytes / (ms_sep * 1e-3) / 1e9},
        threshold_repack={"layer": "512 -> 256 at M=65536 (gemm_mfma_kernel)",
                          "plain_us": statistics.fmean(t_l1) * 1e3,
                          "threshold_flip_us": statistics.fmean(t_l1t) * 1e3,
                          "binary_gops": 2.0 * M * dims[0] * dims[1]
                          / (statistics.fmean(t_l1t) * 1e-3) / 1e9},
        step_inputs=(d, None, None),
    )
    if cpu:
        res["threshold_repack"]["cpu_baseline"] = thr_cpu_baseline(h0, wps[0], thr, flip, dims)
    return res


def small_legs(calib=None, cpu=True):
    """The two latency-bound configurations: gemv_small (M=1, K=512, N=256,
    int32; one bnn_gemv_act launch) and edge_1000 (M=64, K=N=1000: pack X,
    int32 and alpha-scaled products, and the K = 0 repack), each timed as
    back-to-back calls in one HIP graph, with the oracle timed on one
    thread."""
    import torch
    import packed_xor_popcount_amd as bnn
    import workloads
    dev = torch.device("cuda:0")
    out = []
    d = workloads.make("gemv_small")
    K = d["K"]
    x = d["x"].to(dev)
    wp = bnn.pack_signs(d["w"].to(dev))
    y = torch.empty((1, wp.shape[0]), dtype=torch.int32, device=dev)
    ms = graph_ms(lambda: bnn.gemv_act(x, wp, K, bnn.EPI_I32, out=y), 200)
    rec = {"workload": "gemv_small", "us_per_step": ms * 1e3,
           "binary_gops": 2.0 * 256 * K / (ms * 1e-3) / 1e9,
           "step": "bnn_gemv_act (fp32 x packed in-kernel, int32 out)"}
    if cpu:
        rec["cpu_baseline"] = small_cpu("gemv_small", d)
    out.append(rec)
    d = workloads.make("edge_1000")
    K = d["K"]
    x = d["x"].to(dev)
    wp = bnn.pack_signs(d["w"].to(dev))
    alpha = d["alpha"].to(dev)
    M, N = x.shape[0], wp.shape[0]
    xp = torch.empty((M, bnn.words(K)), dtype=torch.int64, device=dev)
    yi = torch.empty((M, N), dtype=torch.int32, device=dev)
    yf = torch.empty((M, N), dtype=torch.float32, device=dev)
    e0 = torch.empty((M, 0), dtype=torch.int64, device=dev)
    w0 = torch.empty((N, 0), dtype=torch.int64, device=dev)
    yr = torch.empty((M, bnn.words(N)), dtype=torch.int64, device=dev)

    def step():
        bnn.pack_signs(x, out=xp)
        bnn.gemm_u64(xp, wp, K, out=yi)
        bnn.gemm_u64_scaled(xp, wp, alpha, K, out=yf)
        bnn.gemm_sign_repack(e0, w0, 0, out=yr)

    ms = graph_ms(step, 100)
    rec = {"workload": "edge_1000", "us_per_step": ms * 1e3,
           "binary_gops": 2 * 2.0 * M * N * K / (ms * 1e-3) / 1e9,
           "step": "pack X + bnn_gemm_u64 + bnn_gemm_u64_scaled + K=0 bnn_gemm_sign_repack"}
    if cpu:
        rec["cpu_baseline"] = small_cpu("edge_1000", d)
    out.append(rec)
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of the workload


def small_cpu(name, d, seconds=1.5):
    """The oracle on one thread, whole steps of a small configuration."""
    import numpy as np
    import oracle
    K = d["K"]
    wp = oracle.pack(d["w"].numpy())
    x = d["x"].numpy()
    n, t0 = 0, time.perf_counter()
    while n < 3 or time.perf_counter() - t0 < seconds:
        xp = oracle.pack(x)
        oracle.gemm_i32(xp, wp, K, nthreads=1)
        if name == "edge_1000":
            oracle.gemm_scaled(xp, wp, d["alpha"].numpy(), K, nthreads=1)
            oracle.sign_repack(np.zeros((x.shape[0], 0), np.uint64),
                               np.zeros((wp.shape[0], 0), np.uint64), 0, nthreads=1)
        n += 1
    dt = (time.perf_counter() - t0) / n
    M, N = x.shape[0], wp.shape[0]
    ops = 2.0 * M * N * K * (2 if name == "edge_1000" else 1)
    return {"value": ops / dt / 1e9, "unit": "binary GOPS", "cores": 1, "kind": "oracle",
            "us_per_step": dt * 1e6, "sample": f"{n} whole steps on one thread"}


def cpu_baseline(workload, step_inputs, seconds):
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


def strip(rec, keys=("step_inputs",)):
    return {k: v for k, v in rec.items() if k not in keys}


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
    cpu = not args.no_cpu_baseline
    wl = args.workload
    defaults = {"gemv_4096": (1024, 64), "gemv_stream": (20, 2), "named_gemv_4096": (1024, 64),
                "ffn_4096": (20, 3), "chain_65536": (50, 5), "signw_gemv_4096": (1024, 64),
                "signw_16384": (50, 5), "small": (1, 0), "calibrate": (1, 0)}
    steps = args.steps if args.steps is not None else defaults[wl][0]
    warmup = args.warmup if args.warmup is not None else defaults[wl][1]
    log(f"[bench] workload={wl} steps={steps} warmup={warmup}")
    nested = wl == "gemv_4096" and not args.no_nested
    calib = None
    if nested or wl == "calibrate":
        calib = calibrate()
        log("[bench] calibration: " + ", ".join(
            f"{k} {v['rate']:.1f} {v['unit']} (sclk {v['sclk_mhz'] or 0:.0f} MHz)"
            for k, v in calib.items() if isinstance(v, dict) and "rate" in v)
            + (f", launch floor {calib['launch_floor']['us']:.2f} us" if "launch_floor" in calib
               else ""))
        if wl == "calibrate":
            print(json.dumps({"metric": METRIC, "calibration": calib}), flush=True)
            return

    if wl in ("gemv_4096", "gemv_stream"):
        res = gemv_leg(steps, warmup, calib, rows=STREAM_ROWS if wl == "gemv_stream" else None,
                       eager=args.eager)
    elif wl == "named_gemv_4096":
        leg = named_gemv_leg(steps, warmup, calib)
        res = dict(leg, config=dict(leg["config"], workload=leg["workload"]), step_inputs=None)
    elif wl == "ffn_4096":
        res = ffn_leg(steps, calib)
    elif wl == "chain_65536":
        res = chain_leg(steps, calib, cpu)
    elif wl == "small":
        recs = small_legs(calib, cpu)
        print(json.dumps({"metric": METRIC, "small": recs}), flush=True)
        return
    else:
        leg = (signw_gemv_leg(steps, warmup, calib, args.eager)
               if wl == "signw_gemv_4096" else signw_gemm_leg(steps, calib))
        res = dict(leg, config=dict(leg["config"], workload=leg["workload"]), step_inputs=None)
    log(f"[bench] {wl}: {res['value']:.1f} {res['unit']}, {res['ms_per_step'] * 1e3:.2f} us/step")

    out = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u64",
        "data": "synthetic (seeded, see workloads.py)", "config": res["config"],
        "roofline": res["roofline"],
    }
    for k in ("binary_gops", "ablation", "unfused", "threshold_repack", "pack_then_gemm"):
        if k in res:
            out[k] = res[k]
    if cpu and res.get("step_inputs") is not None:
        log("[bench] timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(wl, res["step_inputs"], args.cpu_seconds)
    if cpu and wl.startswith("signw"):
        out["cpu_baseline"] = signw_cpu_baseline(wl, args.cpu_seconds)

    if nested:
        # every other record of the path, each with its roofline and oracle
        st = gemv_leg(20, 2, calib, rows=STREAM_ROWS)
        log(f"[bench] streaming: {st['value']:.1f} GB/s, {st['ms_per_step'] * 1e3:.1f} us/step")
        out["streaming"] = {"workload": st["config"]["workload"], "value": st["value"],
                            "unit": st["unit"], "ms_per_step": st["ms_per_step"], "steps": 20,
                            "config": st["config"], "roofline": st["roofline"]}
        nb = named_gemv_leg(steps, warmup, calib)
        log(f"[bench] named batch-1: {nb['value']:.1f} GB/s, {nb['ms_per_step'] * 1e3:.2f} us; "
            f"pack + gemm {nb['pack_then_gemm']['us_per_step']:.2f} us")
        out["named_batch1"] = nb
        sec = ffn_leg(20, calib)
        log(f"[bench] ffn_4096: {sec['value']:.1f} binary GOPS, "
            f"GEMM {sec['roofline']['kernel_avg_us']:.1f} us")
        rec = {"workload": "ffn_4096", **strip(sec, ("step_inputs", "value", "unit",
                                                     "ms_per_step", "config"))}
        rec.update(value=sec["value"], unit=sec["unit"], ms_per_step=sec["ms_per_step"],
                   config=sec["config"])
        if cpu:
            rec["cpu_baseline"] = cpu_baseline("ffn_4096", sec["step_inputs"], 3.0)
        out["secondary"] = rec
        ch = chain_leg(50, calib, cpu)
        log(f"[bench] chain_65536: {ch['value']:.1f} binary GOPS, "
            f"{ch['ms_per_step'] * 1e3:.1f} us fused, {ch['unfused']['us_per_step']:.1f} us "
            "separate")
        crec = {"workload": "chain_65536", **strip(ch)}
        if cpu:
            crec["cpu_baseline"] = cpu_baseline("chain_65536", ch["step_inputs"], 3.0)
        out["chain"] = crec
        out["signw"] = []
        for leg in (signw_gemv_leg(steps, warmup, calib), signw_gemm_leg(50, calib)):
            log(f"[bench] {leg['workload']}: {leg['value']:.1f} {leg['unit']}, "
                f"{leg['ms_per_step'] * 1e3:.2f} us/step")
            if cpu:
                leg["cpu_baseline"] = signw_cpu_baseline(leg["workload"], 3.0)
            out["signw"].append(leg)
        out["small"] = small_legs(calib, cpu)
        out["calibration"] = calib
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
