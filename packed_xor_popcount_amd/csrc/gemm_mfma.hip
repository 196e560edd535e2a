// gemm_mfma.hip -- packed binary GEMM on the gfx950 matrix cores (large M).
//
// The result is the same integer as the XOR + popcount kernels:
// <x_m, w_n> = K - 2 * popcount(x_m XOR w_n) = sum_k x[k] * w[k] over the K
// logical elements, x, w in {+1, -1} ("Binary Math Effectiveness -- why /
// how / when", section 1: the identity is exact, so the plain sum of
// products is the same number).  Section 3 of that page notes that dense
// tensor units usually beat naive bit kernels; on MI355X the FP4 matrix
// rate is about 8x the VALU XOR + popcount issue rate, so for large M the
// sum of products is taken on the matrix cores instead:
//
//  * a packed bit b is an FP4 (e2m1) operand value (+1.0 = 0x2 when b = 0,
//    -1.0 = 0xA when b = 1): the packed bit IS the FP4 sign bit, so no table
//    is needed.  A 32-bit chunk x of a packed row becomes the four operand
//    registers ((x << (3 - r)) & 0x88888888) | 0x22222222, r = 0..3, i.e.
//    register r nibble j holds bit 4j + r.  This permutes the K elements
//    inside the chunk; a dot product does not depend on the order of its
//    terms, and A and B are unpacked by the same rule, so the product is
//    unchanged.  Seven VALU ops unpack 32 elements.
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP4 and unit
//    scales (E8M0 127) accumulates in fp32.  Each product is +-1 (or 0 for a
//    masked pad element), so every partial sum is an integer of magnitude
//    <= K and is exact while K <= 2^24 (the library uses this kernel only
//    then).  The final fp32 accumulator IS the integer dot.
//  * pad elements (k >= K) get zero nibbles in the A operand, so they add
//    nothing whatever the pad bits of either operand hold.
//
// Tiling: block = 4 waves arranged WR x WC; a wave owns RB x CB tiles of
// 32 x 32 outputs.  Per step of 8 words (512 elements of K) each lane loads
// its rows' / columns' words straight from L2 (lanes 0-31: words k0..k0+3;
// lanes 32-63: words k0+4..k0+7; the eight MFMA slices pair the low or high
// halves of those words), unpacks them in registers and issues RB*CB*8
// MFMAs; the next step's words are loaded before the current step's MFMAs.
// Output layout of a 32 x 32 tile (lane l, accumulator register v): column
// l % 32, row 8 (v / 4) + 4 (l / 32) + v % 4.  The repack epilogue ballots
// two neighbouring tiles: the low 32 ballot bits are one row's 32 columns,
// the high 32 bits those of the row 4 below.
#include "../../include/bnn.h"
#include "bnn_internal.h"
#include "fp4_ops.h"

namespace bnn {
namespace {

// Wave arrangement and per-wave tiles of the wide-output configuration.
#ifndef BNN_MFMA_SW
#define BNN_MFMA_SW 8  // words of K per register step
#endif
#ifndef BNN_MFMA_PIN
#define BNN_MFMA_PIN 1  // pin each step's prefetch ahead of the step's MFMAs
#endif
#ifndef BNN_MFMA_SCHED
#define BNN_MFMA_SCHED 0  // VALU ops to interleave after each MFMA (0: compiler's choice)
#endif
#ifndef BNN_MFMA_WR
#define BNN_MFMA_WR 4
#define BNN_MFMA_WC 1
#define BNN_MFMA_RB 2
#define BNN_MFMA_CB 2
#endif


template <int EPI, int WR, int WC, int RB, int CB>
__global__ void __launch_bounds__(256)
    gemm_mfma_kernel(const uint64_t *__restrict__ xp, const uint64_t *__restrict__ wp,
                     const EpiParams ep, void *__restrict__ yv, int M, int N, int K, int kw,
                     int tiles_n) {
  static_assert(WR * WC == 4, "4 waves per block");
  static_assert(!is_repack(EPI) || CB % 2 == 0, "repack pairs 32-column tiles");
  constexpr int BM = WR * RB * 32, BN = WC * CB * 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - (blockIdx.x / tiles_n) * tiles_n;
  const int m0 = tm * BM + (wave / WC) * (RB * 32);
  const int n0 = tn * BN + (wave % WC) * (CB * 32);
  const int h = lane >> 5;    // which word pair of a 4-word step
  const int li = lane & 31;   // row / column within a 32 x 32 tile

  // Row / column pointers, clamped into the matrices (rows past M and
  // columns past N compute garbage that is never stored).
  const uint64_t *arow[RB];
  const uint64_t *bcol[CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    int m = m0 + rb * 32 + li;
    m = m < M ? m : M - 1;
    arow[rb] = xp + (int64_t)m * kw;
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    int n = n0 + cb * 32 + li;
    n = n < N ? n : N - 1;
    bcol[cb] = wp + (int64_t)n * kw;
  }

  // Per-column epilogue operands, fetched before the K loop: the scale, or
  // the threshold as an fp32 bound that is exact against the (exact, |d| <=
  // K <= 2^24) accumulators -- +inf / -inf outside [-K, K] -- and the flip
  // word of each 64-column pair.
  float a_pre[CB];
  uint64_t f_pre[CB / 2 > 0 ? CB / 2 : 1];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = n0 + cb * 32 + li;
    a_pre[cb] = (EPI == BNN_EPI_SCALED && n < N) ? ep.alpha[n] : 0.0f;
    if (EPI == kEpiRepackThr) {
      const int32_t t = thr_of(ep, n, N);
      a_pre[cb] = t >= K ? __builtin_inff() : (t < -K ? -__builtin_inff() : (float)t);
    }
  }
#pragma unroll
  for (int cp = 0; cp < CB / 2; ++cp)
    f_pre[cp] = EPI == kEpiRepackThr ? flip_of(ep, (n0 >> 6) + cp, N) : 0;
  v16f acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  // Steps of kSW = 8 words (512 elements of K): lanes 0-31 hold words
  // k0 .. k0+3 of their row / column, lanes 32-63 words k0+4 .. k0+7; slice
  // q (0..7) pairs half (q & 1) of word (q >> 1) of both lane halves.  A step
  // is "clean" when all its elements are inside K; only the last step can
  // be partial.
  constexpr int kSW = BNN_MFMA_SW, kHW = kSW / 2;
  const int nsteps = (kw + kSW - 1) / kSW;
  const int nclean = (K >> 6) / kSW;

  const uint32_t c8 = 0x88888888u, c2 = 0x22222222u;
  typedef uint64_t ABuf[RB][kHW];
  typedef uint64_t BBuf[CB][kHW];
  auto load_clean = [&](int s, ABuf &a, BBuf &b) {
    const int w = s * kSW + kHW * h;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < kHW; ++i) a[rb][i] = arow[rb][w + i];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < kHW; ++i) b[cb][i] = bcol[cb][w + i];
  };
  auto mma_step = [&](const ABuf &a, const BBuf &b, bool masked, int s) {
    // word i of this lane's half feeds slices 2i (low 32) and 2i+1 (high 32)
#pragma unroll
    for (int i = 0; i < kHW; ++i) {
      v8i ao[2][RB], bo[2][CB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) fp4_operands(a[rb][i], c8, c2, ao[0][rb], ao[1][rb]);
      if (masked) {
        const int64_t e = (int64_t)(s * kSW + kHW * h + i) * 64;
        const uint32_t v0 = valid_bits(e, K), v1 = valid_bits(e + 32, K);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          ao[0][rb] = mask_operand(ao[0][rb], v0);
          ao[1][rb] = mask_operand(ao[1][rb], v1);
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) fp4_operands(b[cb][i], c8, c2, bo[0][cb], bo[1][cb]);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                ao[q][rb], bo[q][cb], acc[rb][cb], kFmtFp4, kFmtFp4, 0, kScaleOne, 0, kScaleOne);
    }
#if BNN_MFMA_SCHED
    // Interleave: one MFMA, then a few VALU ops (the next word's unpack).
#pragma unroll
    for (int j = 0; j < kHW * 2 * RB * CB; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, BNN_MFMA_SCHED, 0);
    }
#endif
  };

  // Two register buffers in ping-pong: the loads of step s+1 are in flight
  // while step s runs.  A scheduling barrier keeps each prefetch ahead of the
  // MFMAs it is meant to overlap (left alone, the scheduler sinks the loads
  // behind most of the step, and the loop head then waits for every load).  Both halves of the pair loop are unconditional (a
  // conditional use would let the compiler sink the prefetch behind the
  // MFMAs); the load past the last clean step re-reads that step (clamped,
  // in bounds, unused).  An odd last step runs after the loop.
  ABuf a0, a1;
  BBuf b0, b1;
  if (nclean > 0) load_clean(0, a0, b0);
  int s = 0;
  for (; s + 1 < nclean; s += 2) {
    load_clean(s + 1, a1, b1);
#if BNN_MFMA_PIN
    __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before the MFMAs
#endif
    mma_step(a0, b0, false, s);
    load_clean(s + 2 < nclean ? s + 2 : nclean - 1, a0, b0);
#if BNN_MFMA_PIN
    __builtin_amdgcn_sched_barrier(0);
#endif
    mma_step(a1, b1, false, s + 1);
  }
  if (s < nclean) mma_step(a0, b0, false, s);
  if (nclean < nsteps) {  // the partial last step: guarded loads, masked A
    const int w = nclean * kSW + kHW * h;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < kHW; ++i) a0[rb][i] = w + i < kw ? arow[rb][w + i] : 0;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < kHW; ++i) b0[cb][i] = w + i < kw ? bcol[cb][w + i] : 0;
    mma_step(a0, b0, true, nclean);
  }

  // Epilogue.  acc[rb][cb][v] is the exact integer dot of row
  // m0 + rb*32 + 8(v/4) + 4h + v%4 and column n0 + cb*32 + li.
  if (is_repack(EPI)) {
    const int nw = (N + 63) >> 6;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cp = 0; cp < CB / 2; ++cp) {
        const int na = n0 + (2 * cp) * 32 + li, nb2 = na + 32;
        const int wi = (n0 >> 6) + cp;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // bit set (-1) where the dot is <= the threshold (0 for the plain repack)
          const uint64_t lo = __builtin_amdgcn_ballot_w64(na < N && acc[rb][2 * cp][v] <= a_pre[2 * cp]);
          const uint64_t hi =
              __builtin_amdgcn_ballot_w64(nb2 < N && acc[rb][2 * cp + 1][v] <= a_pre[2 * cp + 1]);
          const int r0 = m0 + rb * 32 + 8 * (v >> 2) + (v & 3);
          // lane 0 writes row r0, lane 32 writes row r0 + 4
          const int r = r0 + 4 * h;
          const uint64_t word = (h ? ((hi & 0xFFFFFFFF00000000ull) | (lo >> 32))
                                   : ((hi << 32) | (lo & 0xFFFFFFFFull))) ^ f_pre[cp];
          if (li == 0 && r < M && wi < nw) static_cast<uint64_t *>(yv)[(int64_t)r * nw + wi] = word;
        }
      }
  } else {
    // Row r(v) = 8 (v / 4) + v % 4 of a 32-row tile (plus 4h): four row
    // pointers, stepped by 8 rows.  Tiles wholly inside M skip the row test.
    const int64_t ld = N;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int mt = m0 + rb * 32 + 4 * h;  // row of v = 0 for this lane
      const bool full_rows = m0 + rb * 32 + 32 <= M;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int n = n0 + cb * 32 + li;
        if (n >= N) continue;
        const float a = a_pre[cb];
        if (EPI == BNN_EPI_I32) {
          int32_t *p = static_cast<int32_t *>(yv) + (int64_t)mt * ld + n;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int dr = 8 * (v >> 2) + (v & 3);
            if (full_rows || mt + dr < M) p[dr * ld] = (int)acc[rb][cb][v];
          }
        } else {
          float *p = static_cast<float *>(yv) + (int64_t)mt * ld + n;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int dr = 8 * (v >> 2) + (v & 3);
            if (full_rows || mt + dr < M) p[dr * ld] = __fmul_rn(acc[rb][cb][v], a);
          }
        }
      }
    }
  }
}

template <int EPI, int WR, int WC, int RB, int CB>
hipError_t launch_cfg(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y, int M,
                      int N, int K, hipStream_t s) {
  constexpr int BM = WR * RB * 32, BN = WC * CB * 32;
  const int kw = (K + 63) / 64;
  const int tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * tiles_n;
  hipLaunchKernelGGL((gemm_mfma_kernel<EPI, WR, WC, RB, CB>), dim3((unsigned)tiles), dim3(256), 0,
                     s, xp, wp, ep, y, M, N, K, kw, tiles_n);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y, int M,
                      int N, int K, hipStream_t s) {
  // Narrow outputs stack the four waves along M so that no wave idles.
  if (N <= 64) return launch_cfg<EPI, 4, 1, 1, 2>(xp, wp, ep, y, M, N, K, s);  // 128 x 64
  return launch_cfg<EPI, BNN_MFMA_WR, BNN_MFMA_WC, BNN_MFMA_RB, BNN_MFMA_CB>(xp, wp, ep, y, M, N, K,
                                                                          s);
}

}  // namespace

hipError_t launch_gemm_mfma(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y,
                            int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s) {
  switch (epilogue) {
    case BNN_EPI_I32:
      return launch_epi<BNN_EPI_I32>(xp, wp, ep, y, (int)M, (int)N, (int)K, s);
    case BNN_EPI_SCALED:
      return launch_epi<BNN_EPI_SCALED>(xp, wp, ep, y, (int)M, (int)N, (int)K, s);
    case kEpiRepackThr:
      return launch_epi<kEpiRepackThr>(xp, wp, ep, y, (int)M, (int)N, (int)K, s);
    default:
      return launch_epi<BNN_EPI_REPACK>(xp, wp, ep, y, (int)M, (int)N, (int)K, s);
  }
}

}  // namespace bnn
