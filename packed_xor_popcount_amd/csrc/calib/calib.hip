// calib.hip -- rate probes behind include/bnn_calib.h: register-only loops
// of the two instruction kinds the packed product runs on (the VALU XOR +
// popcount pair and the FP4 matrix-core MFMA), timed against both device
// counters so that the benchmark can report fractions of the rates this
// GPU actually sustains next to the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/bnn.h"
#include "../../../include/bnn_calib.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bcnt_acc(uint32_t v, uint32_t acc) {
  uint32_t r;
  asm volatile("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(acc));  // kept in order
  return r;
}

__device__ __forceinline__ void stamp(int64_t *rec, bool start) {
  const int64_t c = (int64_t)__builtin_amdgcn_s_memtime();
  const int64_t w = (int64_t)__builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    rec[start ? 0 : 1] = c;
    rec[start ? 2 : 3] = w;
  }
}

__global__ void __launch_bounds__(256) calib_valu_kernel(int64_t *out, int64_t iters) {
  int64_t *rec = out + 4 * (int64_t)blockIdx.x;
  const uint32_t t = threadIdx.x + 977u * blockIdx.x;
  uint32_t x[8], a[8];
  uint32_t k[4];
#pragma unroll
  for (int rep = 0; rep < 4; ++rep) k[rep] = (0x9E3779B9u * (rep + 1)) ^ t;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = t * (2 * j + 1);
    a[j] = 0;
  }
  __syncthreads();
  stamp(rec, true);
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int rep = 0; rep < 4; ++rep)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] ^= k[rep];
        a[j] = bcnt_acc(x[j], a[j]);
      }
  }
  stamp(rec, false);
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j] ^ x[j];
  if (s == 0x12345678u) out[4 * (int64_t)gridDim.x] = s;  // keeps the loop live
}

// A 32-bit mix of x (an integer hash; only its bits matter here).
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// PM1 false: the four MFMAs of an iteration share one operand pair whose
// FP4 +1.0 (0x2) / -1.0 (0xA) nibbles vary by lane only.  PM1 true: four
// operand pairs of pseudo-random +-1 nibbles, and MFMA c of an iteration
// takes A set c and B set c + 1 (mod 4), so that every MFMA sees another
// +-1 pattern than the one before it, as in the packed product.
template <bool PM1>
__global__ void __launch_bounds__(256) calib_mfma_kernel(int64_t *out, int64_t iters) {
  int64_t *rec = out + 4 * (int64_t)blockIdx.x;
  const uint32_t lane = threadIdx.x & 63;
  v8i a[4], b[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t ha = PM1 ? mix32(lane * 97u + c * 13u + r * 7u + 1u) : lane * 0x01010101u;
      const uint32_t hb = PM1 ? mix32(lane * 89u + c * 31u + r * 5u + 1000u) : lane * 0x10101010u;
      a[c][r] = r < 4 ? (int)(0x22222222u | (ha & 0x88888888u)) : 0;
      b[c][r] = r < 4 ? (int)(0x22222222u | (hb & 0x88888888u)) : 0;
    }
  v16f acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  __syncthreads();
  stamp(rec, true);
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          a[PM1 ? c : 0], b[PM1 ? (c + 1) & 3 : 0], acc[c], 4, 4, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
  }
  stamp(rec, false);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  if (s == 1.2345f) out[4 * (int64_t)gridDim.x] = (int64_t)s;  // keeps the loop live
}

// Streaming read of `units` 16-byte units: each block step reads a
// contiguous chunk of 256 x 8 units (32 KiB, eight loads in flight per
// thread), and the blocks stride over the chunks; the folded value keeps
// every load live.  (Eight loads per thread spread a grid stride apart read
// about 15 % slower: more DRAM pages open at once.)
__global__ void __launch_bounds__(256)
    calib_read_kernel(const u32x4 *__restrict__ src, int64_t units, int64_t *out) {
  int64_t *rec = out + 4 * (int64_t)blockIdx.x;
  constexpr int kU = 8;
  constexpr int64_t kChunk = 256 * kU;
  uint32_t f = 0;
  stamp(rec, true);
  int64_t base = (int64_t)blockIdx.x * kChunk;
  for (; base + kChunk <= units; base += (int64_t)gridDim.x * kChunk) {
    u32x4 v[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) v[j] = __builtin_nontemporal_load(src + base + j * 256 + threadIdx.x);
#pragma unroll
    for (int j = 0; j < kU; ++j) f ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // the last partial chunk (units not a multiple of the chunk)
  for (int64_t i = base + threadIdx.x; base < units && i < units; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    f ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  stamp(rec, false);
  if (f == 0x9E3779B9u) out[4 * (int64_t)gridDim.x] = f;  // keeps the loads live
}

int check(const int64_t *out, int64_t blocks, int64_t iters) {
  if (!out) return BNN_E_NULL;
  if (blocks <= 0 || iters <= 0 || blocks >= (int64_t(1) << 30)) return BNN_E_SHAPE;
  if ((uintptr_t)out % 8) return BNN_E_ALIGN;
  return BNN_OK;
}

}  // namespace

extern "C" {

int bnn_calib_valu(int64_t *out, int64_t blocks, int64_t iters, void *stream) {
  const int st = check(out, blocks, iters);
  if (st != BNN_OK) return st;
  hipLaunchKernelGGL(calib_valu_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? BNN_OK : BNN_E_LAUNCH;
}

int bnn_calib_mfma_fp4(int64_t *out, int64_t blocks, int64_t iters, void *stream) {
  const int st = check(out, blocks, iters);
  if (st != BNN_OK) return st;
  hipLaunchKernelGGL(calib_mfma_kernel<false>, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? BNN_OK : BNN_E_LAUNCH;
}

int bnn_calib_mfma_fp4_pm1(int64_t *out, int64_t blocks, int64_t iters, void *stream) {
  const int st = check(out, blocks, iters);
  if (st != BNN_OK) return st;
  hipLaunchKernelGGL(calib_mfma_kernel<true>, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? BNN_OK : BNN_E_LAUNCH;
}

int bnn_calib_read(const void *src, int64_t bytes, int64_t *out, int64_t blocks, void *stream) {
  const int st = check(out, blocks, 1);
  if (st != BNN_OK) return st;
  if (bytes <= 0 || bytes % 16) return BNN_E_SHAPE;
  if (!src) return BNN_E_NULL;
  if ((uintptr_t)src % 16) return BNN_E_ALIGN;
  hipLaunchKernelGGL(calib_read_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src), bytes / 16,
                     out);
  return hipGetLastError() == hipSuccess ? BNN_OK : BNN_E_LAUNCH;
}

int64_t bnn_calib_wallclock_hz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return (int64_t)khz * 1000;
}

}  // extern "C"
