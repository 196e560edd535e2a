// sign_bits.h -- device helpers that turn real values into packed sign bits,
// shared by the packer and the fused activation-packing GEMV.
//
// "Binary Math Effectiveness -- why / how / when", section 1: a value > 0
// projects to +1 (bit 0), anything else to -1 (bit 1); pad bits are 0.
// The test is done on the bit pattern so that flush-to-zero can never flip a
// sign: an fp32 pattern b is > 0 exactly when 0 < (int32)b <= 0x7F800000
// (positive subnormal, normal or +inf), i.e. (b - 1) < 0x7F800000 unsigned;
// -0, +0, NaN and negatives are not.  bf16 is the upper half of an fp32
// pattern, so the same test applies to its 16 bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bnn {

__device__ __forceinline__ uint32_t minus_f32(uint32_t b) { return (b - 1u) >= 0x7F800000u; }
__device__ __forceinline__ uint32_t minus_bf16(uint32_t h) {
  return ((h - 1u) & 0xFFFFu) >= 0x7F80u;
}

// Sign byte of the 8 elements starting at flat element index e0 of `src`
// (DT 0: fp32, 1: bf16): element e -> bit e.  Only the first n_ok (0..8)
// elements exist; the others are not read and give 0 (pad) bits.  VEC: the
// 8 elements are 16-byte aligned, read with 16-byte loads when all exist.
template <int DT, bool VEC>
__device__ __forceinline__ uint32_t sign_byte(const void *src, int64_t e0, int n_ok) {
  uint32_t b = 0;
  if (VEC && n_ok == 8) {
    if (DT == 0) {
      const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint32_t *>(src) + e0);
      const uint4 a = p[0], c = p[1];
      b = minus_f32(a.x) | minus_f32(a.y) << 1 | minus_f32(a.z) << 2 | minus_f32(a.w) << 3 |
          minus_f32(c.x) << 4 | minus_f32(c.y) << 5 | minus_f32(c.z) << 6 | minus_f32(c.w) << 7;
    } else {
      const uint4 a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + e0);
      b = minus_bf16(a.x & 0xFFFFu) | minus_bf16(a.x >> 16) << 1 | minus_bf16(a.y & 0xFFFFu) << 2 |
          minus_bf16(a.y >> 16) << 3 | minus_bf16(a.z & 0xFFFFu) << 4 |
          minus_bf16(a.z >> 16) << 5 | minus_bf16(a.w & 0xFFFFu) << 6 | minus_bf16(a.w >> 16) << 7;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e < n_ok) {
        const uint32_t v = DT == 0 ? static_cast<const uint32_t *>(src)[e0 + e]
                                   : (uint32_t) static_cast<const uint16_t *>(src)[e0 + e];
        b |= (DT == 0 ? minus_f32(v) : minus_bf16(v)) << e;
      }
    }
  }
  return b;
}

// Assemble the bytes of 8 consecutive lanes (lane & 7 == t holds the byte for
// bits 8t .. 8t+7) into one 64-bit word.  Every lane of the wave must call it
// (it shuffles); the word is valid in the lane with t == 0.
__device__ __forceinline__ uint64_t word_from_bytes(uint32_t byte, int t) {
  uint32_t v = byte << (8 * (t & 3));
  v |= __shfl_xor(v, 1, 64);
  v |= __shfl_xor(v, 2, 64);
  const uint32_t hi = __shfl_xor(v, 4, 64);
  return (uint64_t)v | ((uint64_t)hi << 32);
}

}  // namespace bnn
