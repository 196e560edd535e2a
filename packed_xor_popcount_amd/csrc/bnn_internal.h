// bnn_internal.h -- declarations shared by the HIP translation units of
// libbnn.so (kernel launchers and small device helpers).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bnn.h"

namespace bnn {

// Mask of the logical bits of a row's last 64-bit word.
__host__ __device__ inline uint64_t tail_mask(int64_t k) {
  const int r = (int)(k & 63);
  return r ? ((uint64_t(1) << r) - 1) : ~uint64_t(0);
}

// Epilogue selector beyond the public ones: sign -> repack against a
// per-channel threshold, with an optional flip mask (bnn_gemm_sign_repack_thr).
constexpr int kEpiRepackThr = 3;
__host__ __device__ constexpr bool is_repack(int epi) {
  return epi == BNN_EPI_REPACK || epi == kEpiRepackThr;
}

// Per-output-channel epilogue operands (each used by one epilogue only).
struct EpiParams {
  const float *alpha;    // [N] fp32 scales (BNN_EPI_SCALED)
  const int32_t *thr;    // [N] thresholds (kEpiRepackThr)
  const uint64_t *flip;  // [words(N)] flip mask or null (kEpiRepackThr)
};

// Launchers: each enqueues its kernel(s) on `s` and returns hipGetLastError().
// Arguments are already validated by the C-ABI layer.
hipError_t launch_pack(const void *src, int dtype, int64_t rows, int64_t k, int64_t ld,
                       uint64_t *dst, hipStream_t s);

hipError_t launch_gemm_tiled(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y,
                             int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s);

// Matrix-core (FP4 MFMA) GEMM; exact while K <= 2^24.
hipError_t launch_gemm_mfma(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y,
                            int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s);

hipError_t launch_gemv(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y,
                       int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s);

// GEMV whose activation rows arrive as fp32 (dtype 0) or bf16 (dtype 1)
// values, row stride ldx elements, and are sign-packed inside the kernel.
hipError_t launch_gemv_act(const void *x, int dtype, int64_t ldx, const uint64_t *wp,
                           const EpiParams &ep, void *y, int64_t M, int64_t N, int64_t K,
                           int epilogue, hipStream_t s);

// Real-valued bf16 activations times packed sign weights (bnn_gemm_signw_bf16):
// y[m][n] = alpha[n] * sum_k x[m][k] * w_n[k]; alpha may be null (no scale).
// The GEMV form (small M) holds the activation rows in LDS, at most this many
// bytes; signw_gemv_fits tells whether a shape qualifies.
constexpr size_t kSignwGemvMaxLds = 64 * 1024;
size_t signw_gemv_lds_bytes(int64_t M, int64_t kw, int vec);
bool signw_gemv_fits(int64_t M, int64_t K);
hipError_t launch_signw_gemv(const uint16_t *x, int64_t ldx, const uint64_t *wp,
                             const float *alpha, float *y, int64_t M, int64_t N, int64_t K,
                             hipStream_t s);
hipError_t launch_signw_mfma(const uint16_t *x, int64_t ldx, const uint64_t *wp,
                             const float *alpha, float *y, int64_t M, int64_t N, int64_t K,
                             hipStream_t s);

// Three chained binary layers in one launch (bnn_chain3): pack real rows
// (dtype 0 fp32, 1 bf16), two sign -> repack layers, one fp32 layer.  The
// packed weights of all three layers and each wave's hidden rows live in
// LDS, at most this many bytes.
constexpr int64_t kChain3MaxLds = 64 * 1024;
// Optional threshold repack of the two hidden layers (null: plain).
struct Chain3Repack {
  const int32_t *thr1;
  const uint64_t *flip1;
  const int32_t *thr2;
  const uint64_t *flip2;
};
bool chain3_dims_ok(int64_t K0, int64_t N1, int64_t N2, int64_t N3);
hipError_t launch_chain3(const void *x, int dtype, int64_t ldx, const uint64_t *w1,
                         const uint64_t *w2, const uint64_t *w3, const float *alpha, float *y,
                         int64_t M, int64_t K0, int64_t N1, int64_t N2, int64_t N3,
                         const Chain3Repack &rp, hipStream_t s);

// Threshold-repack operands, loaded by the kernels before their K loops from
// clamped (always in-bounds) indexes: the threshold of output column n, and
// the flip word of 64-column group wi with its bits past column N cleared
// (so that pad bits of the output stay 0).
__device__ __forceinline__ int32_t thr_of(const EpiParams &ep, int64_t n, int64_t N) {
  return ep.thr[n < N ? n : N - 1];
}
__device__ __forceinline__ uint64_t flip_of(const EpiParams &ep, int64_t wi, int64_t N) {
  if (!ep.flip) return 0;
  const int64_t nw = (N + 63) >> 6;
  return wi < nw - 1 ? ep.flip[wi] : (ep.flip[nw - 1] & tail_mask(N));
}

constexpr int kWave = 64;  // CDNA wavefront width

// s_waitcnt operand: wait until no vector memory operation is outstanding
// (the other counters unconstrained).  Kernels issue it once before an
// epilogue of many stores whose values depend on earlier loads: with
// nothing outstanding the stores need no waits, whereas the compiler,
// losing track of such loads across the stores' branches, would otherwise
// wait for every earlier store before each new one.
constexpr int kWaitVmem0 = 0x0F70;

// A copy of a loaded value that the compiler treats as computed at this
// point: taking it waits for the load once (for exactly that load), and
// later uses of the copy -- inside loops, behind branches -- need no wait
// on vector memory, so they never drain loads or stores issued after it.
// Register-only.
__device__ __forceinline__ uint32_t settled(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}
__device__ __forceinline__ uint64_t settled(uint64_t v) {
  return (uint64_t)settled((uint32_t)v) | ((uint64_t)settled((uint32_t)(v >> 32)) << 32);
}
constexpr int64_t kMfmaMaxK = int64_t(1) << 24;  // fp32 accumulation of +-1 is exact up to here

// acc + popcount(v) as the single accumulate form of v_bcnt_u32_b32.  Written
// out so that the compiler cannot reassociate a chain of popcount sums into
// v_add3_u32 trees (one extra VALU op per two words).  Register-only: no
// memory operand.
__device__ __forceinline__ uint32_t popc_acc(uint32_t v, uint32_t acc) {
  uint32_t r;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(acc));
  return r;
}

// Sum of v over aligned groups of L lanes (L a power of two, 1..64); every
// lane of a group receives the group total.  Within a row of 16 lanes the
// exchanges are DPP moves (quad permutes, half-row and row mirrors: VALU
// latency); only the steps across rows use ds_swizzle / a lane permute.
template <int L>
__device__ __forceinline__ uint32_t group_sum(uint32_t v) {
  if (L >= 2) v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  if (L >= 4) v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  if (L >= 8) v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  if (L >= 16) v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false); // row_mirror
  if (L >= 32) v += (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);              // lane ^ 16
  if (L >= 64) v += (uint32_t)__shfl_xor((int)v, 32, 64);
  return v;
}

}  // namespace bnn
