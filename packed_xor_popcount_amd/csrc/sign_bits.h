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

// Sign byte of 8 loaded elements: element e -> bit e (1 when it projects to
// -1), from packed arithmetic instead of one compare per element:
//  * bf16 (two per dword): t = h - 1 (wrapping), u = t + 0x80 saturating at
//    0xFFFF, both as packed 16-bit ops; u >= 0x8000 exactly when
//    t >= 0x7F80, i.e. when the value is not > 0.  So the projection bit of
//    each element is the most significant bit of its half.
//  * fp32: the same with t = b - 1, u = t + 0x00800000 saturating at
//    0xFFFFFFFF: the bit is the most significant bit of u.
// v_perm_b32 then gathers the four bytes that carry those bits into one
// dword, and a multiply collects the four bits (bit 7, 15, 23, 31) into the
// low nibble: ((x & 0x80808080) >> 7) * 0x00204081 puts them at bits 21..24
// with no carries in between.
typedef unsigned short bnn_u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t msb_nibble(uint32_t x) {
  const uint32_t t = (x & 0x80808080u) >> 7;
  return ((t * 0x00204081u) >> 21) & 0xFu;
}

__device__ __forceinline__ uint32_t bf16_pair_minus(uint32_t d) {
  const bnn_u16x2 h = __builtin_bit_cast(bnn_u16x2, d);
  const bnn_u16x2 one = {1, 1}, bias = {0x80, 0x80};
  const bnn_u16x2 u = __builtin_elementwise_add_sat(h - one, bias);
  return __builtin_bit_cast(uint32_t, u);  // bits 15 and 31
}

__device__ __forceinline__ uint32_t f32_minus(uint32_t b) {
  return __builtin_elementwise_add_sat(b - 1u, 0x00800000u);  // bit 31
}

template <int DT>
__device__ __forceinline__ uint32_t byte_of(const Raw8 &r) {
  if (DT == 0) {
    const uint32_t lo = __builtin_amdgcn_perm(f32_minus(r.a.y), f32_minus(r.a.x), 0x0C0C0703u) |
                        __builtin_amdgcn_perm(f32_minus(r.a.w), f32_minus(r.a.z), 0x07030C0Cu);
    const uint32_t hi = __builtin_amdgcn_perm(f32_minus(r.b.y), f32_minus(r.b.x), 0x0C0C0703u) |
                        __builtin_amdgcn_perm(f32_minus(r.b.w), f32_minus(r.b.z), 0x07030C0Cu);
    return msb_nibble(lo) | (msb_nibble(hi) << 4);
  }
  const uint32_t lo = __builtin_amdgcn_perm(bf16_pair_minus(r.a.y), bf16_pair_minus(r.a.x), 0x07050301u);
  const uint32_t hi = __builtin_amdgcn_perm(bf16_pair_minus(r.a.w), bf16_pair_minus(r.a.z), 0x07050301u);
  return msb_nibble(lo) | (msb_nibble(hi) << 4);
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
