// pack.hip -- sign projection + packing along K (bnn_pack_signs).
//
// "Binary Math Effectiveness -- why / how / when", section 1: +1 is stored as
// bit 0 and -1 as bit 1; real inputs project to -1 when <= 0 and to +1 when
// > 0; pad bits encode +1.  Section 2.1: a row of K values is ceil(K/64) words.
//
// Design (gfx950, HBM-bound): eight consecutive lanes build one 64-bit word.
// Lane t of a group reads elements 8t .. 8t+7 of the word with 16-byte
// vector loads (one for bf16, two for fp32), turns them into one byte of
// sign bits (element e -> bit e), and the group ORs its bytes together with
// three xor-shuffles, so lane t's byte lands at bits 8t .. 8t+7 (least
// significant bit first).  A wave therefore covers eight consecutive output
// words per sub-step, which leave as one 64-byte store, and each lane keeps
// kSub sub-steps of loads in flight.  Words of the flattened rows x words(K)
// output are handed out linearly, so short rows (K < 512) pack as densely as
// long ones.  The element of a word past K (the tail) and rows whose start is
// not 16-byte aligned fall back to guarded element loads.
#include "bnn_internal.h"

namespace bnn {
namespace {

// Projection on the bit pattern, so flush-to-zero can never flip a sign.
// fp32: the value is > 0 exactly when 0 < (int32)b <= 0x7F800000 (positive
// subnormal, normal or +inf); -0, +0, NaN and negatives are not.
__device__ __forceinline__ uint32_t minus_f32(uint32_t b) { return (b - 1u) >= 0x7F800000u; }
// bf16 is the upper half of an fp32 pattern: the same test on 16 bits.
__device__ __forceinline__ uint32_t minus_bf16(uint32_t h) { return ((h - 1u) & 0xFFFFu) >= 0x7F80u; }

constexpr int kSub = 4;  // words per lane group in flight

template <int DT>
__device__ __forceinline__ uint32_t load_elem(const void *src, int64_t i) {
  if (DT == 0) return static_cast<const uint32_t *>(src)[i];
  return static_cast<const uint16_t *>(src)[i];
}

// Sign byte of the 8 elements starting at element index `e0` of the flat
// source; `n_ok` of them (0..8) exist, the rest contribute 0 (pad) bits.
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
        const uint32_t v = load_elem<DT>(src, e0 + e);
        b |= (DT == 0 ? minus_f32(v) : minus_bf16(v)) << e;
      }
    }
  }
  return b;
}

template <int DT, bool VEC>
__global__ void __launch_bounds__(256)
    pack_kernel(const void *__restrict__ src, int64_t k, int64_t ld, int64_t kw, int64_t total,
                uint64_t *__restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 3;  // which of the wave's 8 words
  const int t = lane & 7;     // which byte of that word
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const uint32_t ukw = (uint32_t)kw;
  for (int64_t g0 = wave * (8 * kSub); g0 < total; g0 += nwaves * (8 * kSub)) {
    const int64_t row0 = g0 / kw;            // wave-uniform
    const uint32_t w0 = (uint32_t)(g0 - row0 * kw);
    uint32_t byte[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      const uint32_t tw = w0 + (uint32_t)(s * 8 + grp);
      const uint32_t dr = tw / ukw;
      const int64_t row = row0 + dr;
      const int64_t w = tw - dr * ukw;
      const int64_t e = w * 64 + t * 8;      // element index within the row
      int n_ok = 0;
      if (g0 + s * 8 + grp < total) {
        const int64_t left = k - e;
        n_ok = left >= 8 ? 8 : (left > 0 ? (int)left : 0);
      }
      byte[s] = sign_byte<DT, VEC>(src, row * ld + e, n_ok);
    }
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      uint32_t v = byte[s] << (8 * (t & 3));
      v |= __shfl_xor(v, 1, 64);
      v |= __shfl_xor(v, 2, 64);
      const uint32_t hi = __shfl_xor(v, 4, 64);
      const int64_t g = g0 + s * 8 + grp;
      if (t == 0 && g < total) dst[g] = (uint64_t)v | ((uint64_t)hi << 32);
    }
  }
}

template <int DT, bool VEC>
void launch(const void *src, int64_t k, int64_t ld, int64_t kw, int64_t total, uint64_t *dst,
            hipStream_t s) {
  const int64_t waves = (total + 8 * kSub - 1) / (8 * kSub);
  int64_t blocks = (waves + 3) / 4;
  const int64_t cap = 256 * 16;  // grid-stride beyond 16 blocks per CU
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((pack_kernel<DT, VEC>), dim3((unsigned)blocks), dim3(256), 0, s, src, k, ld,
                     kw, total, dst);
}

}  // namespace

hipError_t launch_pack(const void *src, int dtype, int64_t rows, int64_t k, int64_t ld,
                       uint64_t *dst, hipStream_t s) {
  const int64_t kw = (k + 63) / 64;
  const int64_t total = rows * kw;
  if (total == 0) return hipSuccess;
  const int64_t esize = dtype == 0 ? 4 : 2;
  // 16-byte vector loads need every row start (and hence every group of 8
  // elements) 16-byte aligned.
  const bool vec = ((uintptr_t)src % 16 == 0) && ((ld * esize) % 16 == 0 || rows == 1);
  if (dtype == 0) {
    if (vec) launch<0, true>(src, k, ld, kw, total, dst, s);
    else launch<0, false>(src, k, ld, kw, total, dst, s);
  } else {
    if (vec) launch<1, true>(src, k, ld, kw, total, dst, s);
    else launch<1, false>(src, k, ld, kw, total, dst, s);
  }
  return hipGetLastError();
}

}  // namespace bnn
