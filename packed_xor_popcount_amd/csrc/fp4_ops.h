// fp4_ops.h -- packed sign bits as FP4 (e2m1) matrix-core operands, shared
// by the MFMA GEMM and the fused chain kernel.
//
// A packed bit b is the FP4 value +1.0 (0x2) when b = 0 and -1.0 (0xA) when
// b = 1 ("Binary Math Effectiveness -- why / how / when", section 1
// encoding): the packed bit IS the FP4 sign bit.  A 32-bit chunk x becomes
// the four operand registers ((x << (3 - r)) & 0x88888888) | 0x22222222,
// r = 0..3, so register r nibble j holds bit 4j + r.  That permutes K inside
// the chunk; A and B are unpacked by the same rule, so a dot product is
// unchanged.  v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales then sums
// +-1 products exactly in fp32 while K <= 2^24.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bnn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kScaleOne = 0x7F7F7F7F;  // E8M0 127 = 2^0 in every byte
constexpr int kFmtFp4 = 4;             // cbsz / blgp: e2m1

// (a & m) | c as one v_and_or_b32.  gfx9 VOP3 encodings take no literal, so
// the compiler would otherwise emit v_and + v_or with literals; with m and c
// held in VGPRs (hoisted out of every loop) it is one op.  Register-only.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// w << S as one v_lshlrev_b64 (the compiler splits a 64-bit shift whose
// halves are used apart into two 32-bit ops).  `pinned`: volatile, so that
// the scheduler keeps it where it is written.
template <int S>
__device__ __forceinline__ uint64_t shl64(uint64_t w, bool pinned = false) {
  uint64_t r;
  if (pinned)
    asm volatile("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "i"(S), "v"(w));
  else
    asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "i"(S), "v"(w));
  return r;
}

// Operands of both 32-element halves of a packed word w: register r of the
// half's operand is ((half << (3 - r)) & 0x88888888) | 0x22222222.  One
// 64-bit shift serves both halves: the bits it carries from the low half
// into the high half land in bit positions 0..2, which the mask drops.
// Eleven VALU ops for 64 elements.
__device__ __forceinline__ void fp4_operands(uint64_t w, uint32_t c8, uint32_t c2, v8i &lo,
                                             v8i &hi) {
  const uint64_t s1 = shl64<1>(w), s2 = shl64<2>(w), s3 = shl64<3>(w);
  lo[0] = (int)and_or((uint32_t)s3, c8, c2);
  lo[1] = (int)and_or((uint32_t)s2, c8, c2);
  lo[2] = (int)and_or((uint32_t)s1, c8, c2);
  lo[3] = (int)and_or((uint32_t)w, c8, c2);
  hi[0] = (int)and_or((uint32_t)(s3 >> 32), c8, c2);
  hi[1] = (int)and_or((uint32_t)(s2 >> 32), c8, c2);
  hi[2] = (int)and_or((uint32_t)(s1 >> 32), c8, c2);
  hi[3] = (int)and_or((uint32_t)(w >> 32), c8, c2);
  lo[4] = lo[5] = lo[6] = lo[7] = 0;
  hi[4] = hi[5] = hi[6] = hi[7] = 0;
}

// Zero the nibbles of elements whose bit in `valid` is 0 (same permutation
// as fp4_operand).
__device__ __forceinline__ v8i mask_operand(v8i a, uint32_t valid) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t s = (valid << (3 - r)) & 0x88888888u;
    const uint32_t fill = s | (s >> 1) | (s >> 2) | (s >> 3);
    a[r] = (int)((uint32_t)a[r] & fill);
  }
  return a;
}

__device__ __forceinline__ uint32_t valid_bits(int64_t e, int64_t K) {
  if (e >= K) return 0u;
  const int64_t left = K - e;
  return left >= 32 ? 0xFFFFFFFFu : ((1u << left) - 1u);
}

}  // namespace bnn
