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

// Raw bit patterns of 8 consecutive elements (fp32: 8 words; bf16: 8 halves
// packed two per word in lo..hi order).  Loading is split from the sign test
// so that a caller can put several of these loads in flight before using
// any of them.
struct Raw8 {
  uint4 a, b;  // fp32: a = elements 0-3, b = 4-7; bf16: a = elements 0-7
};

// Load the 8 elements starting at flat element index e0 of `src` (DT 0:
// fp32, 1: bf16).  Only the first n_ok (0..8) exist; the others are not read
// and are given the pattern of +1.0 (they become 0, i.e. pad, bits).  VEC:
// the 8 elements are 16-byte aligned and are read with 16-byte loads when all
// of them exist.
template <int DT, bool VEC>
__device__ __forceinline__ Raw8 load_raw8(const void *src, int64_t e0, int n_ok) {
  Raw8 r;
  if (VEC && n_ok == 8) {
    if (DT == 0) {
      const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint32_t *>(src) + e0);
      r.a = p[0];
      r.b = p[1];
    } else {
      r.a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + e0);
      r.b = make_uint4(0, 0, 0, 0);
    }
    return r;
  }
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (DT == 0)
      v[e] = e < n_ok ? static_cast<const uint32_t *>(src)[e0 + e] : 0x3F800000u;
    else
      v[e] = e < n_ok ? (uint32_t) static_cast<const uint16_t *>(src)[e0 + e] : 0x3F80u;
  }
  if (DT == 0) {
    r.a = make_uint4(v[0], v[1], v[2], v[3]);
    r.b = make_uint4(v[4], v[5], v[6], v[7]);
  } else {
    r.a = make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
    r.b = make_uint4(0, 0, 0, 0);
  }
  return r;
}

// Sign byte of 8 loaded elements: element e -> bit e (1 when it projects to -1).
template <int DT>
__device__ __forceinline__ uint32_t byte_of(const Raw8 &r) {
  if (DT == 0)
    return minus_f32(r.a.x) | minus_f32(r.a.y) << 1 | minus_f32(r.a.z) << 2 |
           minus_f32(r.a.w) << 3 | minus_f32(r.b.x) << 4 | minus_f32(r.b.y) << 5 |
           minus_f32(r.b.z) << 6 | minus_f32(r.b.w) << 7;
  return minus_bf16(r.a.x & 0xFFFFu) | minus_bf16(r.a.x >> 16) << 1 |
         minus_bf16(r.a.y & 0xFFFFu) << 2 | minus_bf16(r.a.y >> 16) << 3 |
         minus_bf16(r.a.z & 0xFFFFu) << 4 | minus_bf16(r.a.z >> 16) << 5 |
         minus_bf16(r.a.w & 0xFFFFu) << 6 | minus_bf16(r.a.w >> 16) << 7;
}

// Assemble the bytes of 8 consecutive lanes (lane & 7 == t holds the byte for
// bits 8t .. 8t+7) into one 64-bit word.  Every lane of the wave must call it
// (it exchanges registers across lanes); the word is valid in the lane with
// t == 0.  The exchanges are DPP moves: two quad permutes OR the four bytes
// of each quad into a dword, and a half-row mirror hands lane 0 of the group
// the dword of lanes 4-7 (from lane 7).
__device__ __forceinline__ uint64_t word_from_bytes(uint32_t byte, int t) {
  uint32_t v = byte << (8 * (t & 3));
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // half mirror
  return (uint64_t)v | ((uint64_t)hi << 32);
}

}  // namespace bnn
