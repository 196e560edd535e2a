// bnn_internal.h -- declarations shared by the HIP translation units of
// libbnn.so (kernel launchers and small device helpers).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bnn {

// Launchers: each enqueues its kernel(s) on `s` and returns hipGetLastError().
// Arguments are already validated by the C-ABI layer.
hipError_t launch_pack(const void *src, int dtype, int64_t rows, int64_t k, int64_t ld,
                       uint64_t *dst, hipStream_t s);

hipError_t launch_gemm_tiled(const uint64_t *xp, const uint64_t *wp, const float *alpha, void *y,
                             int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s);

// Matrix-core (FP4 MFMA) GEMM; exact while K <= 2^24.
hipError_t launch_gemm_mfma(const uint64_t *xp, const uint64_t *wp, const float *alpha, void *y,
                            int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s);

hipError_t launch_gemv(const uint64_t *xp, const uint64_t *wp, const float *alpha, void *y,
                       int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s);

// GEMV whose activation rows arrive as fp32 (dtype 0) or bf16 (dtype 1)
// values, row stride ldx elements, and are sign-packed inside the kernel.
hipError_t launch_gemv_act(const void *x, int dtype, int64_t ldx, const uint64_t *wp,
                           const float *alpha, void *y, int64_t M, int64_t N, int64_t K,
                           int epilogue, hipStream_t s);

// Mask of the logical bits of a row's last 64-bit word.
__host__ __device__ inline uint64_t tail_mask(int64_t k) {
  const int r = (int)(k & 63);
  return r ? ((uint64_t(1) << r) - 1) : ~uint64_t(0);
}

constexpr int kWave = 64;  // CDNA wavefront width
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
