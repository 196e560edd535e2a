// gemm_tiled.hip -- LDS-tiled XOR + popcount GEMM (large M).
//
// Computes d[m][n] = popcount over the K logical bits of (x_m XOR w_n) and
// then <x_m, w_n> = K - 2d ("Binary Math Effectiveness -- why / how / when",
// section 1, the core identity in its XOR form; the edge-case table's
// "logical n" rule is the masked last word).  Epilogues: int32, one fp32
// multiply by alpha[n], or the projected sign packed along N for the next
// binary layer.
//
// Design for gfx950 (VALU-issue bound: per 32 bits of K and per output, one
// v_xor_b32 and one v_bcnt_u32_b32 that also accumulates):
//  * block = 4 wavefronts; tile = 32 rows x 256 columns.  Wave v owns rows
//    m0 + 8v .. m0 + 8v + 7 (wave-uniform: X words are LDS broadcast reads);
//    lane l owns columns n0 + l + 64c, c = 0..3, so stores are
//    coalesced and each group of 64 consecutive columns sits in one wave
//    (one ballot makes a repacked word).
//  * W and X are staged through LDS in chunks of 8 words (512 bits) of K: 256
//    columns x 64 B, rows padded to 80 B (an odd multiple of 16 B) so the
//    16-byte reads of 64 consecutive columns are bank-conflict free.
//  * register block 8 x 4 outputs per lane: each 16-byte LDS read feeds 32
//    XOR + 32 popcount-accumulate instructions.
//  * the last word of K is masked in both operands when staged; words past
//    the end of K, rows past M and columns past N read as 0 and are never
//    stored.
#include "../../include/bnn.h"
#include "bnn_internal.h"

namespace bnn {
namespace {

constexpr int kRowsPerWave = 8;
constexpr int kWaves = 4;
constexpr int kBM = kRowsPerWave * kWaves;  // 32
constexpr int kColsPerLane = 4;
constexpr int kBN = 64 * kColsPerLane;  // 256
constexpr int kKC = 8;                  // words of K per LDS chunk
constexpr int kLdsStride = kKC * 8 + 16;  // bytes per staged column

__device__ __forceinline__ uint64_t load_word(const uint64_t *__restrict__ p, int64_t row,
                                              int64_t kw, int64_t kk, uint64_t tmask) {
  if (kk >= kw) return 0;
  const uint64_t v = p[row * kw + kk];
  return kk == kw - 1 ? (v & tmask) : v;
}

template <int EPI>
__global__ void __launch_bounds__(256)
    gemm_tiled_kernel(const uint64_t *__restrict__ xp, const uint64_t *__restrict__ wp,
                      const EpiParams ep, void *__restrict__ yv, int M, int N, int K, int kw,
                      int tiles_n, int64_t tiles) {
  __shared__ __attribute__((aligned(16))) unsigned char wl[kBN * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint64_t xl[kBM][kKC];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
  const int tm = (int)(tile / tiles_n);
  const int tn = (int)(tile - (int64_t)tm * tiles_n);
  const int m0 = tm * kBM + wave * kRowsPerWave;
  const int n0 = tn * kBN;
  const uint64_t tmask = tail_mask(K);

  // Scales (or thresholds and flip words) of this lane's columns, fetched
  // before the K loop (on gfx9 the vector-memory counter also counts stores,
  // so a load between the epilogue's stores would make later waits drain
  // them).
  float a_pre[kColsPerLane];
  int32_t t_pre[kColsPerLane];
  uint64_t f_pre[kColsPerLane];
#pragma unroll
  for (int c = 0; c < kColsPerLane; ++c) {
    const int n = n0 + lane + 64 * c;
    a_pre[c] = (EPI == BNN_EPI_SCALED && n < N) ? ep.alpha[n] : 0.0f;
    t_pre[c] = EPI == kEpiRepackThr ? thr_of(ep, n, N) : 0;
    f_pre[c] = EPI == kEpiRepackThr ? flip_of(ep, (n0 >> 6) + c, N) : 0;
  }

  uint32_t acc[kRowsPerWave][kColsPerLane];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int c = 0; c < kColsPerLane; ++c) acc[r][c] = 0;

  for (int k0 = 0; k0 < kw; k0 += kKC) {
    __syncthreads();  // the previous chunk has been consumed
    // Stage W[n0 .. n0+255][k0 .. k0+7]: 256 columns x 4 pieces of 16 B.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + i * 256;
      const int col = piece >> 2;
      const int part = piece & 3;
      const int n = n0 + col;
      uint64_t a = 0, b = 0;
      if (n < N) {
        a = load_word(wp, n, kw, k0 + 2 * part, tmask);
        b = load_word(wp, n, kw, k0 + 2 * part + 1, tmask);
      }
      uint4 v;
      v.x = (uint32_t)a;
      v.y = (uint32_t)(a >> 32);
      v.z = (uint32_t)b;
      v.w = (uint32_t)(b >> 32);
      *reinterpret_cast<uint4 *>(wl + col * kLdsStride + part * 16) = v;
    }
    // Stage X[tm*32 .. +31][k0 .. k0+7]: one word per thread.
    {
      const int row = tid >> 3;
      const int m = tm * kBM + row;
      xl[row][tid & 7] = (m < M) ? load_word(xp, m, kw, k0 + (tid & 7), tmask) : 0;
    }
    __syncthreads();

#pragma unroll
    for (int q = 0; q < kKC; q += 2) {
      uint4 wv[kColsPerLane];
#pragma unroll
      for (int c = 0; c < kColsPerLane; ++c)
        wv[c] = *reinterpret_cast<const uint4 *>(wl + (lane + 64 * c) * kLdsStride + q * 8);
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        // Same address in every lane: an LDS broadcast read.
        const uint4 xv = *reinterpret_cast<const uint4 *>(&xl[wave * kRowsPerWave + r][q]);
#pragma unroll
        for (int c = 0; c < kColsPerLane; ++c) {
          uint32_t a = acc[r][c];
          a = popc_acc(xv.x ^ wv[c].x, a);
          a = popc_acc(xv.y ^ wv[c].y, a);
          a = popc_acc(xv.z ^ wv[c].z, a);
          a = popc_acc(xv.w ^ wv[c].w, a);
          acc[r][c] = a;
        }
      }
    }
  }

  // Epilogue: <x, w> = K - 2d (computed mod 2^32; the true value fits int32).
  // Nothing is left in flight, so that no store below waits.
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  const int nw = (N + 63) >> 6;
#pragma unroll
  for (int c = 0; c < kColsPerLane; ++c) {
    const int n = n0 + lane + 64 * c;
    const float a = a_pre[c];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int m = m0 + r;
      if (m >= M) continue;
      const int dot = (int)((uint32_t)K - 2u * acc[r][c]);
      if (EPI == BNN_EPI_I32) {
        if (n < N) static_cast<int32_t *>(yv)[(int64_t)m * N + n] = dot;
      } else if (EPI == BNN_EPI_SCALED) {
        if (n < N) static_cast<float *>(yv)[(int64_t)m * N + n] = __fmul_rn((float)dot, a);
      } else {
        const uint64_t word = __builtin_amdgcn_ballot_w64(n < N && dot <= t_pre[c]) ^ f_pre[c];
        const int wi = (n0 >> 6) + c;
        if (lane == 0 && wi < nw) static_cast<uint64_t *>(yv)[(int64_t)m * nw + wi] = word;
      }
    }
  }
  __syncthreads();  // LDS is restaged by the next tile of this block
  }
}

}  // namespace

hipError_t launch_gemm_tiled(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y,
                             int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s) {
  const int kw = (int)((K + 63) / 64);
  const int tiles_n = (int)((N + kBN - 1) / kBN);
  const int64_t tiles = ((M + kBM - 1) / kBM) * (int64_t)tiles_n;
  const int64_t cap = 1 << 20;  // grid-stride over tiles beyond this
  const dim3 grid((unsigned)(tiles < cap ? tiles : cap)), block(256);
  switch (epilogue) {
    case BNN_EPI_I32:
      hipLaunchKernelGGL(gemm_tiled_kernel<BNN_EPI_I32>, grid, block, 0, s, xp, wp, ep, y, (int)M,
                         (int)N, (int)K, kw, tiles_n, tiles);
      break;
    case BNN_EPI_SCALED:
      hipLaunchKernelGGL(gemm_tiled_kernel<BNN_EPI_SCALED>, grid, block, 0, s, xp, wp, ep, y,
                         (int)M, (int)N, (int)K, kw, tiles_n, tiles);
      break;
    case kEpiRepackThr:
      hipLaunchKernelGGL(gemm_tiled_kernel<kEpiRepackThr>, grid, block, 0, s, xp, wp, ep, y,
                         (int)M, (int)N, (int)K, kw, tiles_n, tiles);
      break;
    default:
      hipLaunchKernelGGL(gemm_tiled_kernel<BNN_EPI_REPACK>, grid, block, 0, s, xp, wp, ep, y,
                         (int)M, (int)N, (int)K, kw, tiles_n, tiles);
      break;
  }
  return hipGetLastError();
}

}  // namespace bnn
