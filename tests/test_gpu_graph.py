"""GPU parity of the library's launches captured in a HIP graph and replayed.

Every entry point enqueues its kernels on the caller's stream and keeps no
host state, allocates nothing and clears nothing with a memset, so a captured
sequence replayed on new inputs must give the oracle's results on every
replay.  Each replay runs on inputs copied into the captured buffers
beforehand, with other eager GPU work between the replays, and every output of
every replay is compared with the oracle ("Binary Math Effectiveness -- why /
how / when", section 1, for the packing and every product; "Encoder /
decoder", BinaryAutoEncoder, for the chain; the binary_nn README's packed-sign
path for the real-activation product, here on integer-valued activations so
that every fp32 partial sum is exact).  Bar: bit-exact."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import packed_xor_popcount_amd as bnn
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 3


def say(*a):
    print(*a, flush=True)


def words_np(t):
    return t.cpu().numpy().view(np.uint64)


def assert_scaled_equal(got, ref):
    nz = ref != 0
    assert np.array_equal(got[nz].view(np.uint32), ref[nz].view(np.uint32))
    assert np.all(got[~nz] == 0)


def test_captured_sequence_matches_oracle_on_every_replay():
    say("graph replay: pack + three products, batch-1 decode, chain, real-activation GEMV")
    g = workloads.generator(4242)
    # static operands (weights and scales): fixed across replays
    M, N, K = 300, 700, 1000
    w = workloads.uniform_pm1(g, N, K)
    alpha = workloads.absmean_alpha(w)
    K2, N2 = 4096, 1000
    w2 = workloads.normal(g, N2, K2)
    alpha2 = workloads.absmean_alpha(w2)
    dims = (512, 256, 128, 64)
    wc = [workloads.normal(g, dims[i + 1], dims[i]) for i in range(3)]
    alpha3 = workloads.absmean_alpha(wc[2])
    Ks, Ns = 1024, 500
    ws = workloads.normal(g, Ns, Ks)
    alpha_s = workloads.absmean_alpha(ws)

    wp = bnn.pack_signs(w.to(DEV))
    wp2 = bnn.pack_signs(w2.to(DEV))
    wpc = [bnn.pack_signs(t.to(DEV)) for t in wc]
    wps = bnn.pack_signs(ws.to(DEV))
    a_d, a2_d, a3_d, as_d = (t.to(DEV) for t in (alpha, alpha2, alpha3, alpha_s))

    # captured input and output buffers
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    xr = torch.zeros((1, K2), dtype=torch.bfloat16, device=DEV)
    xc = torch.zeros((200, dims[0]), dtype=torch.float32, device=DEV)
    xs = torch.zeros((3, Ks), dtype=torch.bfloat16, device=DEV)
    xp = torch.empty((M, bnn.words(K)), dtype=torch.int64, device=DEV)
    y_i = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y_f = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y_r = torch.empty((M, bnn.words(N)), dtype=torch.int64, device=DEV)
    y_1 = torch.empty((1, N2), dtype=torch.float32, device=DEV)
    y_c = torch.empty((200, dims[3]), dtype=torch.float32, device=DEV)
    y_s = torch.empty((3, Ns), dtype=torch.float32, device=DEV)

    def sequence():
        bnn.pack_signs(x, out=xp)
        bnn.gemm_u64(xp, wp, K, out=y_i)
        bnn.gemm_u64_scaled(xp, wp, a_d, K, out=y_f)
        bnn.gemm_sign_repack(xp, wp, K, out=y_r)
        bnn.gemv_act(xr, wp2, K2, bnn.EPI_SCALED, alpha=a2_d, out=y_1)
        bnn.chain3(xc, wpc[0], wpc[1], wpc[2], a3_d, out=y_c)
        bnn.gemm_signw_bf16(xs, wps, Ks, as_d, bnn.ALGO_AUTO, out=y_s)

    sequence()  # eager once before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(DEV)
    cap.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            sequence()
    torch.cuda.synchronize()

    rw, rw2, rws = (oracle.pack(t.numpy()) for t in (w, w2, ws))
    for r in range(REPLAYS):
        say("replay", r)
        # new inputs, copied in eagerly, and unrelated eager work before the replay
        h_x = workloads.uniform_pm1(g, M, K).to(torch.bfloat16)
        h_xr = workloads.normal(g, 1, K2).to(torch.bfloat16)
        h_xc = workloads.normal(g, 200, dims[0])
        h_xs = torch.randint(-8, 9, (3, Ks), generator=g).to(torch.bfloat16)
        for dst, src in ((x, h_x), (xr, h_xr), (xc, h_xc), (xs, h_xs)):
            dst.copy_(src.to(DEV))
        busy = torch.randn((512, 512), generator=g).to(DEV)
        busy = busy @ busy
        graph.replay()
        torch.cuda.synchronize()
        del busy

        rx = oracle.pack(workloads.bf16_bits(h_x))
        assert np.array_equal(words_np(xp), rx), f"pack, replay {r}"
        assert np.array_equal(y_i.cpu().numpy(), oracle.gemm_i32(rx, rw, K)), f"int32, replay {r}"
        assert_scaled_equal(y_f.cpu().numpy(), oracle.gemm_scaled(rx, rw, alpha.numpy(), K))
        assert np.array_equal(words_np(y_r), oracle.sign_repack(rx, rw, K)), f"repack, replay {r}"
        rxr = oracle.pack(workloads.bf16_bits(h_xr))
        assert_scaled_equal(y_1.cpu().numpy(), oracle.gemm_scaled(rxr, rw2, alpha2.numpy(), K2))
        ref_c, _ = oracle.chain(h_xc.numpy(), [t.numpy() for t in wc], alpha3.numpy())
        assert_scaled_equal(y_c.cpu().numpy(), ref_c)
        s = oracle.dot_signw_bf16(workloads.bf16_bits(h_xs), rws, Ks)
        ref_s = (s.astype(np.float32) * alpha_s.numpy()[None, :]).astype(np.float32)
        assert_scaled_equal(y_s.cpu().numpy(), ref_s)
