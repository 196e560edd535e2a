// signw.hip -- real-valued bf16 activations times packed sign weights:
//
//   y[m][n] = alpha[n] * sum_k x[m][k] * w_n[k],   w_n[k] = +1 (bit 0) / -1 (bit 1)
//
// the inference form of a layer whose weights alone are binarised (binary_nn
// README, "Binary Regression" and "Triton Kernel Benchmark": BinaryLinear's
// eval-only packed-sign path; the weight encoding is that of "Binary Math
// Effectiveness -- why / how / when", section 1).  The weights keep their
// 1-bit packed form (32x fewer bytes than fp32, section 2.2 of the same
// page); the activations stay real, so the result is a floating-point sum
// (products exact, fp32 accumulation) rather than an integer.
//
// Both kernels turn two weight bits into a pair of bf16 +-1 values with two
// VALU operations.  For a 32-bit chunk c of a packed row (elements
// 32q .. 32q+31) the pair register for position p (0..15) is
//
//   ((c << (15 - p)) & 0x80008000) | 0x3F803F80
//
// i.e. bf16 +1.0 (0x3F80) in both halves with bit p of c as the sign of the
// low half and bit p+16 as the sign of the high half.  The activations are
// staged in the matching order: the 32-bit word for position p holds
// (x[32q + p], x[32q + p + 16]).  Elements past K are staged as +0, so the
// pad bits of the last word never contribute.
//
//  * gemv_signw_kernel (small M, weight-streaming, VALU): L lanes share one
//    column with coalesced 16-byte W loads; each pair of elements is one
//    v_dot2_f32_bf16 against the activation pair held in LDS; the L partial
//    sums are combined with DPP moves.
//  * gemm_signw_kernel (larger M, matrix cores): v_mfma_f32_32x32x16_bf16
//    with the activation tile staged in LDS (pair order, two tiles, one
//    barrier per step) from buffer loads two steps ahead, and the weight
//    fragments unpacked in registers from the packed words, which every lane
//    loads straight from L2.  Blocks are mapped so that the tiles of one
//    8th of the rows run on one XCD (its L2 then reads those rows once).
#include "../../include/bnn.h"
#include "bnn_internal.h"
#include "fp4_ops.h"

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

namespace bnn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr uint32_t kSignMask = 0x80008000u;
constexpr uint32_t kPlusOnes = 0x3F803F80u;  // bf16 (+1.0, +1.0)

// Pair register of weight bits p and p + 16 of chunk c (see the header).
// The constants come in as VGPR operands (gfx9 VOP3 takes no literal).
__device__ __forceinline__ uint32_t sign_pair(uint32_t c_shifted, uint32_t mask, uint32_t ones) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(c_shifted), "v"(mask), "v"(ones));
  return r;
}

// w << s as one 64-bit shift for a shift count that is a constant after
// unrolling (the switch folds away).  Both 32-bit halves of w come out
// shifted for the pair registers: the bits the shift carries from the low
// half into the high half land below bit s <= 15, under the sign positions
// 15 and 31 that sign_pair keeps.
__device__ __forceinline__ uint64_t shl64_const(uint64_t w, int s) {
  switch (s) {
    case 0: return w;
    case 1: return shl64<1>(w);
    case 2: return shl64<2>(w);
    case 3: return shl64<3>(w);
    case 4: return shl64<4>(w);
    case 5: return shl64<5>(w);
    case 6: return shl64<6>(w);
    case 7: return shl64<7>(w);
    case 8: return shl64<8>(w);
    case 9: return shl64<9>(w);
    case 10: return shl64<10>(w);
    case 11: return shl64<11>(w);
    case 12: return shl64<12>(w);
    case 13: return shl64<13>(w);
    case 14: return shl64<14>(w);
    case 15: return shl64<15>(w);
    default: return w << s;
  }
}

__device__ __forceinline__ float dot2(uint32_t xpair, uint32_t wpair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xpair),
                                         __builtin_bit_cast(bf16x2, wpair), acc, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum of v over aligned groups of L lanes (every lane of a group receives it).
template <int L>
__device__ __forceinline__ float group_sum_f32(float v) {
  if (L >= 2) v += dpp_f32<0xB1>(v);   // quad_perm 1,0,3,2
  if (L >= 4) v += dpp_f32<0x4E>(v);   // quad_perm 2,3,0,1
  if (L >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if (L >= 16) v += dpp_f32<0x140>(v); // row_mirror
  if (L >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  if (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// bf16 element k of row m (k may be past K: then +0).
__device__ __forceinline__ uint32_t x_at(const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                                         int64_t K) {
  return k < K ? (uint32_t)x[m * ldx + k] : 0u;
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel for small M.

constexpr int kGemvRows = 8;          // activation rows per launch of the GEMV form
constexpr int kUnitPadBytes = 16;     // LDS pad per unit (spreads lanes over banks)

template <int L, int VEC, int P, bool SCALED, bool XV8>
__global__ void __launch_bounds__(256)
    gemv_signw_kernel(const uint16_t *__restrict__ x, int64_t ldx, const uint64_t *__restrict__ wp,
                      const float *__restrict__ alpha, float *__restrict__ y, int M, int N, int K,
                      int kw) {
  constexpr int G = 64 / L;
  constexpr int CB = 4 * G * P;
  constexpr int kUnitBytes = VEC * 128 + kUnitPadBytes;  // 2 chunks of 64 B per word
  extern __shared__ __attribute__((aligned(16))) unsigned char xs[];  // [M][units][kUnitBytes]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane / L;
  const int part = lane % L;
  const int units = kw / VEC;
  const int nsteps = (N + CB - 1) / CB;
  const uint32_t mask = kSignMask, ones = kPlusOnes;


  // Operands of one block step (the scales of this lane's columns and its W
  // words of each pass, for units u = part, part + L, ... < units), loaded
  // before they are used from clamped, always in-bounds addresses.
  struct StepRegs {
    float a[P];
    uint64_t w[P][VEC];
  };
  auto load_step = [&](int step, StepRegs &r) {
    const int64_t nb = (int64_t)step * CB;
    int uu = part < units ? part : units - 1;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      int64_t n = nb + (int64_t)(p * 4 + wave) * G + sub;
      n = n < N ? n : N - 1;
      r.a[p] = SCALED ? alpha[n] : 1.0f;
      const uint64_t *src = wp + n * kw + (int64_t)uu * VEC;
      // W is read once per call: non-temporal loads keep it from
      // displacing the staged activations' sources and the scales.
      if (VEC == 2) {
        const u64x2 t = __builtin_nontemporal_load(reinterpret_cast<const u64x2 *>(src));
        r.w[p][0] = t.x;
        r.w[p][VEC - 1] = t.y;
      } else {
        r.w[p][0] = __builtin_nontemporal_load(src);
      }
    }
  };
  auto run_step = [&](int step, const StepRegs &r0) {
    const int64_t nb = (int64_t)step * CB;
    float acc[P][kGemvRows];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int rr = 0; rr < kGemvRows; ++rr) acc[p][rr] = 0.0f;
    for (int u = part; u < units; u += L) {
      uint64_t w[P][VEC];
      if (u == part) {  // the unit whose words were loaded ahead
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int v = 0; v < VEC; ++v) w[p][v] = r0.w[p][v];
      } else {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          int64_t n = nb + (int64_t)(p * 4 + wave) * G + sub;
          n = n < N ? n : N - 1;
          const uint64_t *src = wp + n * kw + (int64_t)u * VEC;
          if (VEC == 2) {
            const u64x2 t = __builtin_nontemporal_load(reinterpret_cast<const u64x2 *>(src));
            w[p][0] = t.x;
            w[p][VEC - 1] = t.y;
          } else {
            w[p][0] = __builtin_nontemporal_load(src);
          }
        }
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        // pair registers of both chunks of word v (16 per chunk and column):
        // one 64-bit shift serves chunk 0 (low half) and chunk 1 (high half)
        uint32_t b2[2][P][16];
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const uint64_t sh = shl64_const(w[p][v], 15 - j);
            b2[0][p][j] = sign_pair((uint32_t)sh, mask, ones);
            b2[1][p][j] = sign_pair((uint32_t)(sh >> 32), mask, ones);
          }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // chunk qi = 2v + h of this unit
          const uint32_t(&b)[P][16] = b2[h];
#pragma unroll
          for (int rr = 0; rr < kGemvRows; ++rr) {
            if (rr >= M) break;
            const unsigned char *xr =
                xs + ((size_t)rr * units + u) * kUnitBytes + (2 * v + h) * 64;
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
              const uint4 xv = *reinterpret_cast<const uint4 *>(xr + 16 * j4);
#pragma unroll
              for (int p = 0; p < P; ++p) {
                float a = acc[p][rr];
                a = dot2(xv.x, b[p][4 * j4 + 0], a);
                a = dot2(xv.y, b[p][4 * j4 + 1], a);
                a = dot2(xv.z, b[p][4 * j4 + 2], a);
                a = dot2(xv.w, b[p][4 * j4 + 3], a);
                acc[p][rr] = a;
              }
            }
          }
        }
      }
    }

#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int rr = 0; rr < kGemvRows; ++rr) {
        if (rr >= M) break;
        acc[p][rr] = group_sum_f32<L>(acc[p][rr]);
      }
    if (part == 0) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int64_t n = nb + (int64_t)(p * 4 + wave) * G + sub;
        if (n >= N) continue;
#pragma unroll
        for (int rr = 0; rr < kGemvRows; ++rr) {
          if (rr >= M) break;
          y[(int64_t)rr * N + n] = SCALED ? __fmul_rn(acc[p][rr], r0.a[p]) : acc[p][rr];
        }
      }
    }
  };

  // Stage the activation rows once per block in pair order: word p of chunk
  // q holds (x[32q + p], x[32q + p + 16]).  Item i builds words 4j .. 4j+3
  // of one chunk (one 16-byte LDS store) from the 8-byte pieces
  // x[32q + 4j .. +3] and x[32q + 16 + 4j .. +3]; pieces that reach past K
  // (or rows that are not 8-byte aligned) are read element by element.
  // A thread loads kStageItems items before it waits on any.  The loads of
  // the first items go out before the first step's W words and scales:
  // loads retire in order, so the staging then waits only for itself while
  // the W words stay in flight across the barrier.
  constexpr int kStageItems = 4;
  const int chunks = units * VEC * 2;
  const int total = M * chunks * 4;
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(x), (short)0, 0x7FFFFFFF, 0x00020000);
  uint32_t pc[kStageItems][4];
  bool fast[kStageItems];
  auto stage_load = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < kStageItems; ++e) {
      const int i = i0 + 256 * e;
      const int j = i & 3;
      const int rq = i >> 2;
      const int m = rq / chunks, q = rq - m * chunks;
      const int64_t k = (int64_t)q * 32 + 4 * j;
      fast[e] = XV8 & (i < total) & (k + 20 <= K);
      if (XV8) {
        // Out-of-range byte offsets (element-wise or absent items) read 0.
        const uint32_t off = fast[e] ? (uint32_t)((m * ldx + k) * 2) : 0x80000000u;
        const v2u lo = __builtin_amdgcn_raw_buffer_load_b64(xres, off, 0, 0);
        const v2u hi = __builtin_amdgcn_raw_buffer_load_b64(xres, off + 32, 0, 0);
        pc[e][0] = lo.x; pc[e][1] = lo.y; pc[e][2] = hi.x; pc[e][3] = hi.y;
      }
    }
  };
  auto stage_store = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < kStageItems; ++e) {
      const int i = i0 + 256 * e;
      if (i < total) {
        const int j = i & 3;
        const int rq = i >> 2;
        const int m = rq / chunks, q = rq - m * chunks;
        const int64_t k = (int64_t)q * 32 + 4 * j;
        if (!fast[e]) {
          pc[e][0] = x_at(x, ldx, m, k, K) | (x_at(x, ldx, m, k + 1, K) << 16);
          pc[e][1] = x_at(x, ldx, m, k + 2, K) | (x_at(x, ldx, m, k + 3, K) << 16);
          pc[e][2] = x_at(x, ldx, m, k + 16, K) | (x_at(x, ldx, m, k + 17, K) << 16);
          pc[e][3] = x_at(x, ldx, m, k + 18, K) | (x_at(x, ldx, m, k + 19, K) << 16);
        }
        uint4 v;
        v.x = __builtin_amdgcn_perm(pc[e][2], pc[e][0], 0x05040100u);
        v.y = __builtin_amdgcn_perm(pc[e][2], pc[e][0], 0x07060302u);
        v.z = __builtin_amdgcn_perm(pc[e][3], pc[e][1], 0x05040100u);
        v.w = __builtin_amdgcn_perm(pc[e][3], pc[e][1], 0x07060302u);
        const int u = q / (VEC * 2), qi = q - u * (VEC * 2);
        *reinterpret_cast<uint4 *>(xs + ((size_t)m * units + u) * kUnitBytes + qi * 64 + j * 16) =
            v;
      }
    }
  };
  stage_load(tid);
  // The first step's operands; later steps run in pairs whose operands are
  // loaded one step ahead (single-step blocks load nothing extra; the
  // register sets are never copied).
  StepRegs ra;
  load_step(blockIdx.x, ra);
  stage_store(tid);
  for (int i0 = tid + 256 * kStageItems; i0 < total; i0 += 256 * kStageItems) {
    stage_load(i0);
    stage_store(i0);
  }
  __syncthreads();
  for (int step = blockIdx.x; step < nsteps; step += 2 * gridDim.x) {
    const int sb = step + gridDim.x, sa = step + 2 * gridDim.x;
    StepRegs rb;
    if (sb < nsteps) load_step(sb, rb);  // uniform
    run_step(step, ra);
    if (sa < nsteps) load_step(sa, ra);
    if (sb < nsteps) run_step(sb, rb);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core kernel.
//
// v_mfma_f32_32x32x16_bf16: lane l supplies row / column l % 32 and, in its
// four registers, 8 of the 16 k values (lanes 0-31 one half, 32-63 the other;
// which k go in which register is free as long as A and B agree).  For the
// 32-element chunk q of a 64-element block step, MFMA t (0, 1), lane half h
// and register j hold the element pair (p, p + 16) with p = 8t + 4h + j.
// The 32 x 32 output layout: lane l, register v -> row 8(v/4) + 4(l/32) +
// v%4, column l%32.

constexpr int kBK = 64;                       // elements of K per block step (one W word)
constexpr int kARowBytes = 2 * 64 + 16;       // two chunks of 64 B + pad

#ifndef BNN_SIGNW_PIN
#define BNN_SIGNW_PIN 1  // keep each step's prefetch ahead of its MFMAs
#endif
// MINB: blocks per CU the register allocation must allow.
template <int WR, int WC, int RB, int CB, int MINB, bool SCALED, bool XV8>
__global__ void __launch_bounds__(256, MINB)
    gemm_signw_kernel(const uint16_t *__restrict__ x, int64_t ldx, const uint64_t *__restrict__ wp,
                      const float *__restrict__ alpha, float *__restrict__ y, int M, int N, int K,
                      int kw, int tiles_m, int tiles_n) {
  static_assert(WR * WC == 4, "4 waves per block");
  constexpr int BM = WR * RB * 32, BN = WC * CB * 32;
  constexpr int kPerThread = BM * 8 / 256;  // 16-byte A fragments staged per thread per step
  static_assert(BM * 8 % 256 == 0, "whole fragments per thread");
  // Two LDS tiles: step s is staged into tile s % 2 while the other one may
  // still be read by step s - 1, so one barrier per step suffices.
  __shared__ __attribute__((aligned(16))) unsigned char as[2][BM * kARowBytes];
  // The weight words of the block's BN columns for the same step, staged
  // beside the activations (thread t loads column t's word two steps ahead,
  // like its activation pieces, and every lane reads its columns' words back):
  // loaded straight into each lane per step instead, the words' latency was
  // exposed at every step.
  static_assert(BN <= 256, "one weight word per thread and step");
  __shared__ __attribute__((aligned(16))) uint64_t ws[2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int li = lane & 31;

  // XCD-aware tile order: hardware places block b on XCD b % 8, so block b
  // takes logical tile (b % 8) * per + b / 8 and each XCD owns a contiguous
  // range of tiles (rows of X are then fetched by one L2).  Grids that are
  // not a multiple of 8 keep the plain order.
  const int nblocks = tiles_m * tiles_n;
  const int per = nblocks >> 3;
  const int tile = (nblocks % 8 == 0) ? (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3)
                                      : (int)blockIdx.x;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * BM + (wave / WC) * (RB * 32);
  const int n0 = tn * BN + (wave % WC) * (CB * 32);

  // Scales of this lane's columns (clamped; columns past N are never stored),
  // and the weight row this thread stages (column tid of the block tile).
  float a_pre[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    int n = n0 + cb * 32 + li;
    n = n < N ? n : N - 1;
    a_pre[cb] = SCALED ? alpha[n] : 1.0f;
  }
  const uint64_t *wrow_t;
  {
    int n = tn * BN + (tid < BN ? tid : BN - 1);
    n = n < N ? n : N - 1;
    wrow_t = wp + (int64_t)n * kw;
  }
  // this wave's first column inside the block tile
  const int wcol = (wave % WC) * (CB * 32);

  // Fragments staged by this thread: f = tid + 256 i is (row f / 8, chunk
  // (f / 4) & 1, t = (f / 2) & 1, h = f & 1) and holds the four pairs
  // (x[b + j], x[b + j + 16]), b = 32 chunk + 8t + 4h.  f % 8 = tid % 8 for
  // every i, so all of a thread's fragments share the offset b and their rows
  // are 32 apart.  Full steps (all 64 elements inside K) read two 8-byte
  // pieces per fragment through a buffer resource: the per-thread byte
  // offset is fixed and the step's offset is a scalar, so a step costs no
  // vector address arithmetic.  The last, partial step (K % 64 != 0) reads
  // element by element with zero fill past K.
  const int koff = 32 * ((tid >> 2) & 1) + 8 * ((tid >> 1) & 1) + 4 * (tid & 1);
  const int frow = tid >> 3;
  int64_t xrow[kPerThread];
  uint32_t voff[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    int64_t m = (int64_t)tm * BM + frow + 32 * i;
    m = m < M - 1 ? m : M - 1;
    xrow[i] = m * ldx + koff;
    voff[i] = (uint32_t)(xrow[i] * 2);
  }
  typedef uint32_t Stage[kPerThread][4];  // lo pair, hi pair of each fragment
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(x), (short)0, 0x7FFFFFFF, 0x00020000);
  auto load_full = [&](int kb, Stage &r) {
    const int soff = kb * kBK * 2;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      if (XV8) {
        const v2u a = __builtin_amdgcn_raw_buffer_load_b64(xres, voff[i], soff, 0);
        const v2u b = __builtin_amdgcn_raw_buffer_load_b64(xres, voff[i] + 32, soff, 0);
        r[i][0] = a.x; r[i][1] = a.y; r[i][2] = b.x; r[i][3] = b.y;
      } else {
        const uint16_t *p = x + xrow[i] + (int64_t)kb * kBK;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          r[i][j] = (uint32_t)p[2 * j] | ((uint32_t)p[2 * j + 1] << 16);
          r[i][2 + j] = (uint32_t)p[16 + 2 * j] | ((uint32_t)p[16 + 2 * j + 1] << 16);
        }
      }
    }
  };
  auto load_tail = [&](int kb, Stage &r) {
    const int64_t k0 = (int64_t)kb * kBK + koff;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const uint16_t *p = x + xrow[i] + (int64_t)kb * kBK;
      uint32_t e[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = k0 + j < K ? (uint32_t)p[j] : 0u;
        e[4 + j] = k0 + 16 + j < K ? (uint32_t)p[16 + j] : 0u;
      }
      r[i][0] = e[0] | (e[1] << 16); r[i][1] = e[2] | (e[3] << 16);
      r[i][2] = e[4] | (e[5] << 16); r[i][3] = e[6] | (e[7] << 16);
    }
  };
  auto store_a = [&](const Stage &r, unsigned char *buf) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      uint4 v;  // pairs j = 0..3: low half from the first piece, high half from the second
      v.x = __builtin_amdgcn_perm(r[i][2], r[i][0], 0x05040100u);
      v.y = __builtin_amdgcn_perm(r[i][2], r[i][0], 0x07060302u);
      v.z = __builtin_amdgcn_perm(r[i][3], r[i][1], 0x05040100u);
      v.w = __builtin_amdgcn_perm(r[i][3], r[i][1], 0x07060302u);
      *reinterpret_cast<uint4 *>(buf + (frow + 32 * i) * kARowBytes + (tid & 7) * 16) = v;
    }
  };

  v16f acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  const uint32_t mask = kSignMask, ones = kPlusOnes;
  const int wrow = (wave / WC) * (RB * 32);  // this wave's first row inside the block tile
  auto compute = [&](const unsigned char *buf, const uint64_t *wbuf) {
    uint64_t wcur[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) wcur[cb] = wbuf[wcol + cb * 32 + li];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // activation fragments of both chunks q (one LDS read each)
      bf16x8 afr[2][RB];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          afr[q][rb] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4 *>(
                          buf + (wrow + rb * 32 + li) * kARowBytes + q * 64 + t * 32 + h * 16));
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        // the column's word, pre-shifted by 4 for lane half 0; one 64-bit
        // shift per pair position gives both chunks' pair registers (what it
        // carries into the high half lands below the sign positions)
        const uint64_t w = h ? wcur[cb] : (wcur[cb] << 4);
        uint32_t r[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint64_t sh = shl64_const(w, 11 - 8 * t - j);
          r[0][j] = sign_pair((uint32_t)sh, mask, ones);
          r[1][j] = sign_pair((uint32_t)(sh >> 32), mask, ones);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const bf16x8 bfr = __builtin_bit_cast(bf16x8, make_uint4(r[q][0], r[q][1], r[q][2], r[q][3]));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[q][rb], bfr, acc[rb][cb], 0, 0, 0);
        }
      }
    }
  };

  // Two register stages in flight over the full steps: while step s is
  // staged and computed, the activation and weight loads of step s + 2 are
  // in flight.  The loop is unrolled by two so that each stage keeps its own
  // registers, and no loaded value is ever copied (a copy waits for its
  // load): a stage's registers are reloaded right after they are written to
  // LDS, the weight word first (the oldest load of a stage is waited for
  // first).  Loads past the last full step re-read it (in bounds, unused).
  const int nfull = K / kBK;
  const int last = nfull - 1;
  Stage ra, rb;
  uint64_t wra = 0, wrb = 0;  // this thread's staged weight word of each stage
  if (nfull > 0) {
    // the issue order pinned (weight word, then activations, stage a then
    // stage b), the same as in the loop, so that the loop head's waits are
    // exact: each waits for its own stage and leaves the other one in flight
    wra = wrow_t[0];
    __builtin_amdgcn_sched_barrier(0);
    load_full(0, ra);
    __builtin_amdgcn_sched_barrier(0);
    const int s1 = last < 1 ? last : 1;
    wrb = wrow_t[s1];
    __builtin_amdgcn_sched_barrier(0);
    load_full(s1, rb);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Whole pairs of steps in the loop (no branch inside it, so that the wait
  // counts the compiler derives at the loop head are exact, not the merge of
  // two paths); an odd last full step, already loaded into stage a, after.
  for (int s = 0; s + 1 < nfull; s += 2) {
    const int s2 = s + 2 < last ? s + 2 : last;
    const int s3 = s + 3 < last ? s + 3 : last;
    store_a(ra, as[0]);
    if (BN == 256 || tid < BN) ws[0][tid] = wra;
    __syncthreads();
    wra = wrow_t[s2];
    __builtin_amdgcn_sched_barrier(0);
    load_full(s2, ra);
#if BNN_SIGNW_PIN
    __builtin_amdgcn_sched_barrier(0);
#endif
    compute(as[0], ws[0]);
    store_a(rb, as[1]);
    if (BN == 256 || tid < BN) ws[1][tid] = wrb;
    __syncthreads();
    wrb = wrow_t[s3];
    __builtin_amdgcn_sched_barrier(0);
    load_full(s3, rb);
#if BNN_SIGNW_PIN
    __builtin_amdgcn_sched_barrier(0);
#endif
    compute(as[1], ws[1]);
  }
  if (nfull & 1) {  // uniform branch; stage a holds step nfull - 1
    store_a(ra, as[0]);
    if (BN == 256 || tid < BN) ws[0][tid] = wra;
    __syncthreads();
    compute(as[0], ws[0]);
  }
  if (nfull < kw) {  // the partial last step, zero past K (uniform branch)
    load_tail(nfull, ra);
    wra = wrow_t[nfull];
    __syncthreads();  // both tiles are free
    store_a(ra, as[0]);
    if (BN == 256 || tid < BN) ws[0][tid] = wra;
    __syncthreads();
    compute(as[0], ws[0]);
  }

  // Nothing is left in flight, so that no store below waits; tiles wholly
  // inside M store without a row test (straight-line stores).
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  const int64_t ld = N;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int mt = m0 + rb * 32 + 4 * h;
    const bool full_rows = m0 + rb * 32 + 32 <= M;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int n = n0 + cb * 32 + li;
      if (n >= N) continue;
      float *p = y + (int64_t)mt * ld + n;
      auto put = [&](int v) __attribute__((always_inline)) {
        p[(int64_t)(8 * (v >> 2) + (v & 3)) * ld] =
            SCALED ? __fmul_rn(acc[rb][cb][v], a_pre[cb]) : acc[rb][cb][v];
      };
      if (full_rows) {
#pragma unroll
        for (int v = 0; v < 16; ++v) put(v);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (mt + 8 * (v >> 2) + (v & 3) < M) put(v);
      }
    }
  }
}

template <int L, int VEC, int P, bool SCALED>
hipError_t launch_gemv_lp(const uint16_t *x, int64_t ldx, const uint64_t *wp, const float *alpha,
                          float *y, int M, int N, int K, int kw, hipStream_t s) {
  // 8-byte activation pieces need 8-byte aligned row starts, and the buffer
  // loads 32-bit byte offsets (all of X below 2 GiB).
  const bool xv8 = ((uintptr_t)x % 8 == 0) && (ldx % 4 == 0 || M == 1) &&
                   ((int64_t)(M - 1) * ldx + K) * 2 < (int64_t(1) << 31);
  constexpr int CB = 4 * (64 / L) * P;
  const int64_t steps = ((int64_t)N + CB - 1) / CB;
  const int64_t cap = 256 * 8;
  const int64_t blocks = steps < cap ? steps : cap;
  const size_t shmem = signw_gemv_lds_bytes(M, kw, VEC);
  if (xv8)
    hipLaunchKernelGGL((gemv_signw_kernel<L, VEC, P, SCALED, true>), dim3((unsigned)blocks),
                       dim3(256), shmem, s, x, ldx, wp, alpha, y, M, N, K, kw);
  else
    hipLaunchKernelGGL((gemv_signw_kernel<L, VEC, P, SCALED, false>), dim3((unsigned)blocks),
                       dim3(256), shmem, s, x, ldx, wp, alpha, y, M, N, K, kw);
  return hipGetLastError();
}

template <int VEC, bool SCALED>
hipError_t launch_gemv_vec(const uint16_t *x, int64_t ldx, const uint64_t *wp, const float *alpha,
                           float *y, int M, int N, int K, int kw, hipStream_t s) {
  const int units = kw / VEC;
#define BNN_SIGNW_L(LL) return launch_gemv_lp<LL, VEC, 1, SCALED>(x, ldx, wp, alpha, y, M, N, K, kw, s);
  if (units <= 4) BNN_SIGNW_L(4)
  if (units <= 8) BNN_SIGNW_L(8)
  if (units <= 16) BNN_SIGNW_L(16)
  if (units <= 32) BNN_SIGNW_L(32)
  BNN_SIGNW_L(64)
#undef BNN_SIGNW_L
}

template <int RB, int CB, int MINB, bool SCALED, bool XV8>
hipError_t launch_mfma_cfg(const uint16_t *x, int64_t ldx, const uint64_t *wp, const float *alpha,
                           float *y, int M, int N, int K, hipStream_t s) {
  constexpr int WR = 2, WC = 2;
  constexpr int BM = WR * RB * 32, BN = WC * CB * 32;
  const int kw = (K + 63) / 64;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_signw_kernel<WR, WC, RB, CB, MINB, SCALED, XV8>),
                     dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, s, x, ldx, wp, alpha, y, M,
                     N, K, kw, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

size_t signw_gemv_lds_bytes(int64_t M, int64_t kw, int vec) {
  const int64_t units = vec == 2 ? kw / 2 : kw;
  return (size_t)(M * units * (vec * 128 + kUnitPadBytes));
}

bool signw_gemv_fits(int64_t M, int64_t K) {
  const int64_t kw = (K + 63) / 64;
  return M >= 1 && M <= kGemvRows && K > 0 && signw_gemv_lds_bytes(M, kw, 1) <= kSignwGemvMaxLds;
}

hipError_t launch_signw_gemv(const uint16_t *x, int64_t ldx, const uint64_t *wp,
                             const float *alpha, float *y, int64_t M, int64_t N, int64_t K,
                             hipStream_t s) {
  const int kw = (int)((K + 63) / 64);
  const bool vec2 = kw % 2 == 0 && ((uintptr_t)wp % 16 == 0);
  if (alpha) {
    return vec2 ? launch_gemv_vec<2, true>(x, ldx, wp, alpha, y, (int)M, (int)N, (int)K, kw, s)
                : launch_gemv_vec<1, true>(x, ldx, wp, alpha, y, (int)M, (int)N, (int)K, kw, s);
  }
  return vec2 ? launch_gemv_vec<2, false>(x, ldx, wp, alpha, y, (int)M, (int)N, (int)K, kw, s)
              : launch_gemv_vec<1, false>(x, ldx, wp, alpha, y, (int)M, (int)N, (int)K, kw, s);
}

hipError_t launch_signw_mfma(const uint16_t *x, int64_t ldx, const uint64_t *wp,
                             const float *alpha, float *y, int64_t M, int64_t N, int64_t K,
                             hipStream_t s) {
  // 8-byte activation loads need 8-byte aligned row starts, and the buffer
  // loads 32-bit byte offsets (all of X below 2 GiB).
  const bool xv8 = ((uintptr_t)x % 8 == 0) && (ldx % 4 == 0 || M == 1) &&
                   ((M - 1) * ldx + K) * 2 < (int64_t(1) << 31);
  // Wide outputs: 128 x 256 block tiles (2 x 4 tiles of 32 x 32 per wave,
  // two blocks per CU); narrow ones: 128 x 128.
  const int m = (int)M, n = (int)N, k = (int)K;
  if (N >= 256) {
    if (alpha)
      return xv8 ? launch_mfma_cfg<2, 4, 2, true, true>(x, ldx, wp, alpha, y, m, n, k, s)
                 : launch_mfma_cfg<2, 4, 2, true, false>(x, ldx, wp, alpha, y, m, n, k, s);
    return xv8 ? launch_mfma_cfg<2, 4, 2, false, true>(x, ldx, wp, alpha, y, m, n, k, s)
               : launch_mfma_cfg<2, 4, 2, false, false>(x, ldx, wp, alpha, y, m, n, k, s);
  }
  if (alpha)
    return xv8 ? launch_mfma_cfg<2, 2, 1, true, true>(x, ldx, wp, alpha, y, m, n, k, s)
               : launch_mfma_cfg<2, 2, 1, true, false>(x, ldx, wp, alpha, y, m, n, k, s);
  return xv8 ? launch_mfma_cfg<2, 2, 1, false, true>(x, ldx, wp, alpha, y, m, n, k, s)
             : launch_mfma_cfg<2, 2, 1, false, false>(x, ldx, wp, alpha, y, m, n, k, s);
}

}  // namespace bnn
