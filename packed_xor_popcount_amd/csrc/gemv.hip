// gemv.hip -- weight-streaming XOR + popcount product for small M (batch-1
// decode and similar).
//
// Same result as the tiled GEMM: <x_m, w_n> = K - 2 * popcount(x_m XOR w_n)
// over the K logical bits ("Binary Math Effectiveness -- why / how / when",
// section 1).  Sections 2.2-2.3 of that page observe that a batch-1 product
// is bound by the bytes of the weights it streams, 1/32 of fp32 once packed;
// this kernel is built to stream the packed W once, at HBM rate.
//
// Design for gfx950 (HBM-bound):
//  * L lanes (a power of two, 4..64) share one column n = one row of W;
//    each lane reads VEC consecutive words (16 B when VEC = 2) per step, so a
//    wave reads G = 64/L whole W rows with fully coalesced loads.
//  * block = 4 wavefronts; one block step covers 4 * G * P columns, the
//    loads of all P passes issued before any popcount; up to 8 activation
//    rows share every W word loaded (rows beyond 8 re-stream W).
//  * partial counts are summed across the L lanes with xor-shuffles, the
//    column totals are gathered in LDS, and the epilogue stores them
//    coalesced (int32 / alpha-scaled fp32) or ballots 64 of them into one
//    repacked word (P is chosen so that a step covers 64 columns).
//  * the last word of K is masked (pad bits never count).
#include "../../include/bnn.h"
#include "bnn_internal.h"

namespace bnn {
namespace {

constexpr int kMR = 8;  // activation rows sharing one pass over W

template <int EPI, int L, int VEC, int P>
__global__ void __launch_bounds__(256)
    gemv_kernel(const uint64_t *__restrict__ xp, const uint64_t *__restrict__ wp,
                const float *__restrict__ alpha, void *__restrict__ yv, int M, int N, int K,
                int kw) {
  constexpr int G = 64 / L;          // columns per wave per pass
  constexpr int CB = 4 * G * P;      // columns per block step
  static_assert(EPI != BNN_EPI_REPACK || CB == 64, "a repack step covers 64 columns");
  __shared__ uint32_t res[kMR][CB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane / L;
  const int part = lane % L;
  const int units = kw / VEC;  // VEC == 2 only when kw is even
  const uint64_t tmask = tail_mask(K);
  const int64_t nb = (int64_t)blockIdx.x * CB;
  const int nw = (N + 63) >> 6;

  for (int mb = 0; mb < M; mb += kMR) {
    const int mrows = (M - mb) < kMR ? (M - mb) : kMR;
    uint32_t acc[P][kMR];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int r = 0; r < kMR; ++r) acc[p][r] = 0;

    for (int ub = 0; ub < units; ub += L) {
      const int u = ub + part;
      uint64_t w[P][VEC];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int64_t n = nb + (int64_t)(p * 4 + wave) * G + sub;
        const bool ok = (u < units) && (n < N);
#pragma unroll
        for (int v = 0; v < VEC; ++v) w[p][v] = 0;
        if (ok) {
          const uint64_t *src = wp + n * kw + (int64_t)u * VEC;
          if (VEC == 2) {
            const ulonglong2 t = *reinterpret_cast<const ulonglong2 *>(src);
            w[p][0] = t.x;
            w[p][VEC - 1] = t.y;
          } else {
            w[p][0] = src[0];
          }
        }
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const int word = u * VEC + v;
        const uint64_t wm = (word == kw - 1) ? tmask : ~uint64_t(0);
#pragma unroll
        for (int r = 0; r < kMR; ++r) {
          if (r >= mrows) break;
          const uint64_t x = (u < units) ? (xp[(int64_t)(mb + r) * kw + word] & wm) : 0;
#pragma unroll
          for (int p = 0; p < P; ++p) acc[p][r] += (uint32_t)__popcll(x ^ (w[p][v] & wm));
        }
      }
    }

    // Sum the L partial counts of each column (all lanes of a group end with the total).
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int r = 0; r < kMR; ++r) {
        if (r >= mrows) break;
        uint32_t a = acc[p][r];
#pragma unroll
        for (int off = L / 2; off >= 1; off >>= 1) a += __shfl_xor(a, off, 64);
        acc[p][r] = a;
      }
    __syncthreads();  // res is free (previous row block finished its epilogue)
    if (part == 0) {
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int r = 0; r < kMR; ++r) {
          if (r >= mrows) break;
          res[r][(p * 4 + wave) * G + sub] = acc[p][r];
        }
    }
    __syncthreads();

    if (EPI == BNN_EPI_REPACK) {
      if (wave == 0) {
        const int64_t n = nb + lane;
        for (int r = 0; r < mrows; ++r) {
          const int dot = (int)((uint32_t)K - 2u * res[r][lane]);
          const uint64_t word = __builtin_amdgcn_ballot_w64(n < N && dot <= 0);
          if (lane == 0 && (nb >> 6) < nw)
            static_cast<uint64_t *>(yv)[(int64_t)(mb + r) * nw + (nb >> 6)] = word;
        }
      }
    } else {
      for (int i = tid; i < mrows * CB; i += 256) {
        const int r = i / CB, c = i - r * CB;
        const int64_t n = nb + c;
        if (n >= N) continue;
        const int dot = (int)((uint32_t)K - 2u * res[r][c]);
        const int64_t o = (int64_t)(mb + r) * N + n;
        if (EPI == BNN_EPI_I32)
          static_cast<int32_t *>(yv)[o] = dot;
        else
          static_cast<float *>(yv)[o] = __fmul_rn((float)dot, alpha[n]);
      }
    }
  }
}

template <int EPI, int L, int VEC>
hipError_t launch_l(const uint64_t *xp, const uint64_t *wp, const float *alpha, void *y, int M,
                    int N, int K, int kw, hipStream_t s) {
  constexpr int P = (EPI == BNN_EPI_REPACK) ? L / 4 : 1;
  constexpr int CB = 4 * (64 / L) * P;
  const int64_t blocks = ((int64_t)N + CB - 1) / CB;
  hipLaunchKernelGGL((gemv_kernel<EPI, L, VEC, P>), dim3((unsigned)blocks), dim3(256), 0, s, xp,
                     wp, alpha, y, M, N, K, kw);
  return hipGetLastError();
}

template <int EPI, int VEC>
hipError_t launch_vec(const uint64_t *xp, const uint64_t *wp, const float *alpha, void *y, int M,
                      int N, int K, int kw, hipStream_t s) {
  const int units = kw / VEC;
  if (units <= 4) return launch_l<EPI, 4, VEC>(xp, wp, alpha, y, M, N, K, kw, s);
  if (units <= 8) return launch_l<EPI, 8, VEC>(xp, wp, alpha, y, M, N, K, kw, s);
  if (units <= 16) return launch_l<EPI, 16, VEC>(xp, wp, alpha, y, M, N, K, kw, s);
  if (units <= 32) return launch_l<EPI, 32, VEC>(xp, wp, alpha, y, M, N, K, kw, s);
  return launch_l<EPI, 64, VEC>(xp, wp, alpha, y, M, N, K, kw, s);
}

template <int EPI>
hipError_t launch_epi(const uint64_t *xp, const uint64_t *wp, const float *alpha, void *y, int M,
                      int N, int K, int kw, hipStream_t s) {
  const bool vec2 = (kw % 2 == 0) && ((uintptr_t)xp % 16 == 0) && ((uintptr_t)wp % 16 == 0);
  if (vec2) return launch_vec<EPI, 2>(xp, wp, alpha, y, M, N, K, kw, s);
  return launch_vec<EPI, 1>(xp, wp, alpha, y, M, N, K, kw, s);
}

}  // namespace

hipError_t launch_gemv(const uint64_t *xp, const uint64_t *wp, const float *alpha, void *y,
                       int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s) {
  const int kw = (int)((K + 63) / 64);
  switch (epilogue) {
    case BNN_EPI_I32:
      return launch_epi<BNN_EPI_I32>(xp, wp, alpha, y, (int)M, (int)N, (int)K, kw, s);
    case BNN_EPI_SCALED:
      return launch_epi<BNN_EPI_SCALED>(xp, wp, alpha, y, (int)M, (int)N, (int)K, kw, s);
    default:
      return launch_epi<BNN_EPI_REPACK>(xp, wp, alpha, y, (int)M, (int)N, (int)K, kw, s);
  }
}

}  // namespace bnn
