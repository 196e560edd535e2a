// pack.hip -- sign projection + packing along K (bnn_pack_signs).
//
// "Binary Math Effectiveness -- why / how / when", section 1: +1 is stored as
// bit 0 and -1 as bit 1; real inputs project to -1 when <= 0 and to +1 when
// > 0; pad bits encode +1.  Section 2.1: a row of K values is ceil(K/64) words.
//
// Design (gfx950, HBM-bound): a wavefront builds 64 consecutive output words
// of the flattened rows x words(K) output.  For each word, lane i loads
// element 64*w + i of that word's row (one coalesced 256 B / 128 B load per
// word for fp32 / bf16) and the wave-wide ballot of "projects to -1" IS the
// word, with lane i -> bit i (least significant bit first).  Lane j keeps
// word j, so the 64 words leave in one coalesced 512 B store.  Sixteen loads
// are issued before their ballots to keep enough bytes in flight.
#include "bnn_internal.h"

namespace bnn {
namespace {

// Projection on the bit pattern, so flush-to-zero can never flip a sign.
// fp32: the value is > 0 exactly when 0 < (int32)b <= 0x7F800000 (positive
// subnormal, normal or +inf); -0, +0, NaN and negatives are not.
__device__ __forceinline__ bool is_minus_f32(uint32_t b) { return (b - 1u) >= 0x7F800000u; }
// bf16 is the upper half of an fp32 pattern: the same test on 16 bits.
__device__ __forceinline__ bool is_minus_bf16(uint32_t b) { return ((b - 1u) & 0xFFFFu) >= 0x7F80u; }

constexpr uint32_t kPlusOneF32 = 0x3F800000u;  // +1.0f: a lane with no element
constexpr uint32_t kPlusOneBF16 = 0x3F80u;     // contributes a 0 (pad) bit

constexpr int kBatch = 16;  // loads in flight per lane before their ballots

template <int DT>
__global__ void __launch_bounds__(256)
    pack_kernel(const void *__restrict__ src_, int64_t k, int64_t ld, int64_t kw, int64_t total,
                uint64_t *__restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t g0 = wave * 64; g0 < total; g0 += nwaves * 64) {
    int64_t row = g0 / kw;
    int64_t w = g0 - row * kw;
    uint64_t mine = 0;
    for (int jb = 0; jb < 64; jb += kBatch) {
      uint32_t raw[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t col = w * 64 + lane;
        const bool ok = (g0 + jb + j < total) && (col < k);
        if (DT == 0) {
          const uint32_t *src = static_cast<const uint32_t *>(src_);
          raw[j] = ok ? src[row * ld + col] : kPlusOneF32;
        } else {
          const uint16_t *src = static_cast<const uint16_t *>(src_);
          raw[j] = ok ? (uint32_t)src[row * ld + col] : kPlusOneBF16;
        }
        if (++w == kw) {
          w = 0;
          ++row;
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const bool minus = (DT == 0) ? is_minus_f32(raw[j]) : is_minus_bf16(raw[j]);
        const uint64_t word = __builtin_amdgcn_ballot_w64(minus);
        mine = (lane == jb + j) ? word : mine;
      }
    }
    if (g0 + lane < total) dst[g0 + lane] = mine;
  }
}

}  // namespace

hipError_t launch_pack(const void *src, int dtype, int64_t rows, int64_t k, int64_t ld,
                       uint64_t *dst, hipStream_t s) {
  const int64_t kw = (k + 63) / 64;
  const int64_t total = rows * kw;
  if (total == 0) return hipSuccess;
  const int64_t groups = (total + 63) / 64;        // one wave per 64 words
  int64_t blocks = (groups + 3) / 4;                // 4 waves per block
  const int64_t cap = 256 * 8;                      // 8 blocks per CU, grid-stride beyond
  if (blocks > cap) blocks = cap;
  if (dtype == 0)
    hipLaunchKernelGGL(pack_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, src, k, ld, kw,
                       total, dst);
  else
    hipLaunchKernelGGL(pack_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, src, k, ld, kw,
                       total, dst);
  return hipGetLastError();
}

}  // namespace bnn
