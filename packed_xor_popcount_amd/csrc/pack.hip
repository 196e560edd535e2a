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
#include "sign_bits.h"

namespace bnn {
namespace {

constexpr int kSub = 4;  // words per lane group in flight

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
    Raw8 raw[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) {  // all loads first
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
      raw[s] = load_raw8<DT, VEC>(src, row * ld + e, n_ok);
    }
    uint32_t byte[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) byte[s] = byte_of<DT>(raw[s]);
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      const uint64_t word = word_from_bytes(byte[s], t);
      const int64_t g = g0 + s * 8 + grp;
      if (t == 0 && g < total) dst[g] = word;
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
