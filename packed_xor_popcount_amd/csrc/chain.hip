// chain.hip -- a chain of three binary layers in one launch.
//
// Real-valued input rows are sign-projected and packed, the first two
// layers end in sign -> repack (their packed outputs are the next layer's
// input), and the last layer ends alpha-scaled in fp32: the binary MLP /
// auto-encoder stack of chained binary layers ("Encoder / decoder",
// BinaryAutoEncoder; balanced_ternary_engine README, the 512 -> 256 -> 128
// -> 64 example).  The result is bit-identical to bnn_pack_signs followed by
// bnn_gemm_sign_repack twice and bnn_gemm_u64_scaled ("Binary Math
// Effectiveness -- why / how / when", section 1, for every step).
//
// What fusing saves: the packed hidden activations (here 2 + 1 MiB for 65536
// rows) never leave the chip, there is one launch instead of four, and the
// fp32 input is read once while the matrix cores work on earlier rows.
//
// Design for gfx950: one wave owns 32 rows from input to output.
//  * The packed weights of all three layers (21 KiB for 512 -> 256 -> 128 ->
//    64) are copied into LDS once per block, behind the first input loads.
//  * The wave packs its 32 input rows (eight lanes per 64-bit word, as the
//    stand-alone packer does) one K step at a time: step b packs the two
//    words that lanes 0-31 and 32-63 feed to the matrix cores in step b,
//    and the layer-1 MFMAs of step b run while step b + 1's loads are in
//    flight, accumulating the first 128 columns across the steps.
//  * Every layer runs on the matrix cores: v_mfma_scale_f32_32x32x64_f8f6f4
//    with the packed bits as FP4 +-1 operands (exact integer sums).  Lane l
//    holds row / column l % 32 and half l / 32 of its words.
//  * The repack epilogue ballots the signs of two neighbouring 32-column
//    tiles into 64-bit words (as the GEMM does) and writes them to LDS as
//    the next layer's rows; the last layer stores alpha-scaled fp32.
//    Optional per-column thresholds and flip masks make each hidden layer's
//    projection a folded BatchNorm ("Architecture Decision Record",
//    Decision: BN after the binary layers), as bnn_gemm_sign_repack_thr.
#include "../../include/bnn.h"
#include "bnn_internal.h"
#include "fp4_ops.h"
#include "sign_bits.h"

namespace bnn {
namespace {

constexpr int kRows = 32;       // rows per wave
constexpr int kMaxW = 8;        // words of K per layer (K <= 512)
#ifndef BNN_CHAIN_PIPE
#define BNN_CHAIN_PIPE 4
#endif
#ifndef BNN_CHAIN_MIN_BLOCKS
#define BNN_CHAIN_MIN_BLOCKS 2
#endif
// Weight words each thread loads in one go before the first input batch
// (12 x 256 covers 512 -> 256 -> 128 -> 64; larger weights load the rest
// after it).
constexpr int kWeightLoads = 12;
// Layer-1 column tiles accumulated while the input streams in (their
// accumulators stay live across the K steps; 4 keeps two waves per SIMD).
constexpr int kPipeTiles = BNN_CHAIN_PIPE;

// Packed signs of two neighbouring 32 x 32 tiles (columns 64 wi .. 64 wi + 63)
// into the 64-bit words of the wave's 32 rows: out[r * nw + wi].
// acc[v]: row 8 (v / 4) + 4 h + v % 4, column li (+ 32 for the second tile);
// the low ballot bits are row r's 32 columns, the high bits those of row r + 4.
// Each ballot half is written into lane r (or r + 4) of a register pair, so
// that lane r ends up holding row r's word and one store of lanes 0-31
// writes all 32 words.  A bit is set where the exact dot is <= the column's
// bound (tb: the layer's per-column thresholds as exact fp32 bounds, 0
// without thresholds), then the group's flip word is applied.
// v with lane L set to s (wave-uniform).
template <int L>
__device__ __forceinline__ int write_lane(int v, uint32_t s) {
  asm("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(s), "n"(L));
  return v;
}

// Ballots of accumulator register V of both tiles into lanes r and r + 4 of
// lo / hi (r = 8 (V / 4) + V % 4), then the next register.
template <int V>
__device__ __forceinline__ void repack_rows(const v16f &t0, const v16f &t1, float b0, float b1,
                                            int &lo, int &hi) {
  if constexpr (V < 16) {
    constexpr int r = 8 * (V >> 2) + (V & 3);
    const uint64_t m0 = __builtin_amdgcn_ballot_w64(t0[V] <= b0);
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(t1[V] <= b1);
    lo = write_lane<r>(lo, (uint32_t)m0);
    hi = write_lane<r>(hi, (uint32_t)m1);
    lo = write_lane<r + 4>(lo, (uint32_t)(m0 >> 32));
    hi = write_lane<r + 4>(hi, (uint32_t)(m1 >> 32));
    repack_rows<V + 1>(t0, t1, b0, b1, lo, hi);
  }
}

template <bool THR>
__device__ __forceinline__ void repack_pair(const v16f &t0, const v16f &t1, uint64_t *out, int nw,
                                            int wi, int lane, const float *tb, const uint64_t *fw) {
  const int li = lane & 31;
  const float b0 = THR ? tb[64 * wi + li] : 0.0f, b1 = THR ? tb[64 * wi + 32 + li] : 0.0f;
  int lo = 0, hi = 0;  // lane r < 32: row r's word, columns 0-31 / 32-63
  repack_rows<0>(t0, t1, b0, b1, lo, hi);
  const uint64_t f = THR ? fw[wi] : 0;
  if (lane < kRows) out[lane * nw + wi] = (((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo) ^ f;
}

// Columns n_begin .. N-1 of one layer for the wave's 32 rows.  a: the wave's
// packed rows in LDS (stride kw words); w: N x kw packed weights in LDS.
// REPACK: packed signs go to `out` (LDS, stride N / 64 words); otherwise
// fp32 outputs (times alpha[n] when alpha is non-null) go to rows row0.. of
// y (those < M).  Lane l holds row / column l % 32 and, of each operand's
// words, the half l / 32.
// alpha (fp32 outputs) is the scales' copy in LDS, or null for no scale:
// reading it from LDS keeps the stores below free of waits on vector
// memory (a scale register loaded from global memory makes the compiler
// drain every earlier store before each new one).
template <bool REPACK, bool THR>
__device__ __forceinline__ void chain_layer(const uint64_t *a, int kw, const uint64_t *w, int N,
                                            int n_begin, uint64_t *out, const float *tb,
                                            const uint64_t *fw, const float *alpha,
                                            float *__restrict__ y, int64_t row0, int M, int lane) {
  const int h = lane >> 5, li = lane & 31;
  const int hw = kw >> 1;  // words per lane half (kw is even)
  const uint32_t c8 = 0x88888888u, c2 = 0x22222222u;
  v8i ao[kMaxW];
#pragma unroll
  for (int i = 0; i < kMaxW / 2; ++i)
    if (i < hw) fp4_operands(a[li * kw + h * hw + i], c8, c2, ao[2 * i], ao[2 * i + 1]);

  constexpr int TP = REPACK ? 2 : 1;  // 32-column tiles per pass
  for (int n0 = n_begin; n0 < N; n0 += 32 * TP) {
    float a_n = 1.0f;
    if (!REPACK && alpha) a_n = alpha[n0 + li];
    v16f acc[TP];
#pragma unroll
    for (int t = 0; t < TP; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxW / 2; ++i) {
      if (i >= hw) break;
#pragma unroll
      for (int t = 0; t < TP; ++t) {
        v8i bo0, bo1;
        fp4_operands(w[(n0 + 32 * t + li) * kw + h * hw + i], c8, c2, bo0, bo1);
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ao[2 * i], bo0, acc[t], kFmtFp4,
                                                                kFmtFp4, 0, kScaleOne, 0, kScaleOne);
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ao[2 * i + 1], bo1, acc[t],
                                                                kFmtFp4, kFmtFp4, 0, kScaleOne, 0,
                                                                kScaleOne);
      }
    }
    if (REPACK) {
      repack_pair<THR>(acc[0], acc[TP - 1], out, N >> 6, n0 >> 6, lane, tb, fw);
    } else {
      // rows row0 + 8 (v / 4) + v % 4 + 4h; a wave whose 32 rows all exist
      // stores without a row test (straight-line stores)
      float *yp = y + (row0 + 4 * h) * N + n0 + li;
      auto put = [&](int v) __attribute__((always_inline)) {
        yp[(int64_t)(8 * (v >> 2) + (v & 3)) * N] = alpha ? __fmul_rn(acc[0][v], a_n) : acc[0][v];
      };
      if (row0 + kRows <= M) {
#pragma unroll
        for (int v = 0; v < 16; ++v) put(v);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (row0 + 8 * (v >> 2) + (v & 3) + 4 * h < M) put(v);
      }
    }
  }
}

// LDS words: the three packed weight matrices, the two hidden layers'
// repack bounds (fp32, two per word) and flip words, the last layer's
// scales (fp32, two per word), then per wave its packed rows of the input
// and of the two hidden layers.
__host__ __device__ inline int64_t chain3_lds_words(int64_t K0, int64_t N1, int64_t N2,
                                                    int64_t N3) {
  const int64_t kw0 = K0 >> 6, kw1 = N1 >> 6, kw2 = N2 >> 6;
  return N1 * kw0 + N2 * kw1 + N3 * kw2 + (N1 + N2) / 2 + kw1 + kw2 + N3 / 2 +
         4 * kRows * (kw0 + kw1 + kw2);
}

// Repack bound of a hidden column: the threshold as an fp32 value that is
// exact against the exact (|d| <= K) accumulators, +-inf outside [-K, K];
// 0 (the plain projection) without thresholds.
__device__ __forceinline__ float repack_bound(const int32_t *thr, int n, int K) {
  if (!thr) return 0.0f;
  const int32_t t = thr[n];
  return t >= K ? __builtin_inff() : (t < -K ? -__builtin_inff() : (float)t);
}

// THR: the hidden layers repack against thresholds / flip masks.
template <int DT, bool VEC, bool THR>
__global__ void __launch_bounds__(256, BNN_CHAIN_MIN_BLOCKS)
    chain3_kernel(const void *__restrict__ x, int64_t ldx, const uint64_t *__restrict__ w1,
                  const uint64_t *__restrict__ w2, const uint64_t *__restrict__ w3,
                  const float *__restrict__ alpha, float *__restrict__ y, int M, int K0, int N1,
                  int N2, int N3, const Chain3Repack rp) {
  extern __shared__ __attribute__((aligned(16))) uint64_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31, g = lane >> 3, t = lane & 7;
  const int kw0 = K0 >> 6, kw1 = N1 >> 6, kw2 = N2 >> 6;
  const int hw0 = kw0 >> 1;
  const int nw1 = N1 * kw0, nw2 = N2 * kw1, nw3 = N3 * kw2;
  uint64_t *W1 = lds, *W2 = W1 + nw1, *W3 = W2 + nw2;
  float *TB1 = reinterpret_cast<float *>(W3 + nw3), *TB2 = TB1 + N1;
  uint64_t *FW1 = W3 + nw3 + (N1 + N2) / 2, *FW2 = FW1 + kw1;
  float *AL = reinterpret_cast<float *>(FW2 + kw2);
  uint64_t *h0 = FW2 + kw2 + N3 / 2 + wave * kRows * (kw0 + kw1 + kw2);
  uint64_t *h1 = h0 + kRows * kw0, *h2 = h1 + kRows * kw1;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * kRows;
  const uint32_t c8 = 0x88888888u, c2 = 0x22222222u;

  // Input batch b = words b and hw0 + b of the wave's 32 rows (64 words):
  // slot q -> row q / 2, word (q % 2) hw0 + b; lane group g builds slots
  // 8j + g.  Lanes 0-31 of an MFMA take word b of their row, lanes 32-63
  // word hw0 + b, so batch b feeds exactly the layer-1 MFMAs of step b.
  // Element offset of slot j's first element in step 0 (rows clamped into
  // [0, M)); step b adds 64 b.
  int64_t slot0[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = 8 * j + g;
    int64_t m = row0 + (q >> 1);
    m = m < M ? m : M - 1;
    slot0[j] = m * ldx + (int64_t)((q & 1) * hw0) * 64 + 8 * t;
  }
  auto load_batch = [&](int b, Raw8(&raw)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) raw[j] = load_raw8<DT, VEC>(x, slot0[j] + 64 * b, 8);
  };
  auto pack_batch = [&](int b, const Raw8(&raw)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = 8 * j + g;
      const uint64_t word = word_from_bytes(byte_of<DT>(raw[j]), t);
      if (t == 0) h0[(q >> 1) * kw0 + (q & 1) * hw0 + b] = word;
    }
  };

  // The weights of all three layers into LDS (block-wide).  Their loads go
  // out first, all at once (at most kWeightLoads words per thread): the
  // first input batch, issued right behind them, then queues after the
  // weights rather than the weights after the whole grid's first batches.
  Raw8 raw[8];
  {
    const int total = nw1 + nw2 + nw3;
    // word i of the three matrices back to back (a word past them re-reads
    // the last one and is not stored): one unconditional load each, so
    // that all of them are in flight together
    auto word_at = [&](int i) __attribute__((always_inline)) {
      const int j = i < total ? i : total - 1;
      const uint64_t *p = j < nw1 ? w1 + j : (j < nw1 + nw2 ? w2 + (j - nw1) : w3 + (j - nw1 - nw2));
      return *p;
    };
    uint64_t v[kWeightLoads];
#pragma unroll
    for (int u = 0; u < kWeightLoads; ++u) v[u] = word_at(u * 256 + tid);
    // the last layer's scales (N3 <= 512), likewise ahead of the input
    float al[2] = {0.0f, 0.0f};
    if (alpha) {
#pragma unroll
      for (int u = 0; u < 2; ++u) al[u] = alpha[u * 256 + tid < N3 ? u * 256 + tid : N3 - 1];
    }
    load_batch(0, raw);
#pragma unroll
    for (int u = 0; u < kWeightLoads; ++u) {
      const int i = u * 256 + tid;
      if (i < total) lds[i] = v[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (alpha && u * 256 + tid < N3) AL[u * 256 + tid] = al[u];
    // larger weights: the rest word by word
    for (int i = kWeightLoads * 256 + tid; i < total; i += 256) lds[i] = word_at(i);
    // repack bounds and flip words of the hidden layers
    for (int i = tid; THR && i < N1 + N2; i += 256)
      TB1[i] = i < N1 ? repack_bound(rp.thr1, i, K0) : repack_bound(rp.thr2, i - N1, N1);
    for (int i = tid; THR && i < kw1 + kw2; i += 256) {
      const uint64_t *f = i < kw1 ? rp.flip1 : rp.flip2;
      const int wi = i < kw1 ? i : i - kw1, n = i < kw1 ? N1 : N2;
      uint64_t fv = f ? f[wi] : 0;
      if (f && wi == ((n + 63) >> 6) - 1 && (n & 63)) fv &= (uint64_t(1) << (n & 63)) - 1;
      FW1[i] = fv;
    }
  }
  __syncthreads();

  // Pack the input step by step; each step's layer-1 MFMAs (first
  // kPipeTiles column tiles) run while the next step's loads are in flight.
  const int nt1 = N1 >> 5;
  const int np = nt1 < kPipeTiles ? nt1 : kPipeTiles;
  v16f acc[kPipeTiles];
#pragma unroll
  for (int c = 0; c < kPipeTiles; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  for (int b = 0; b < hw0; ++b) {
    pack_batch(b, raw);
    if (b + 1 < hw0) load_batch(b + 1, raw);
    // batch b's words are in LDS: written and read back by this wave only
    // (its own rows), and a wave's LDS accesses take effect in program
    // order, so the wave waits for no other
    __builtin_amdgcn_wave_barrier();
    v8i a0, a1;
    fp4_operands(h0[li * kw0 + h * hw0 + b], c8, c2, a0, a1);
#pragma unroll
    for (int c = 0; c < kPipeTiles; ++c) {
      if (c >= np) break;
      v8i bo0, bo1;
      fp4_operands(W1[(c * 32 + li) * kw0 + h * hw0 + b], c8, c2, bo0, bo1);
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bo0, acc[c], kFmtFp4, kFmtFp4,
                                                              0, kScaleOne, 0, kScaleOne);
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bo1, acc[c], kFmtFp4, kFmtFp4,
                                                              0, kScaleOne, 0, kScaleOne);
    }
  }
#pragma unroll
  for (int cp = 0; cp < kPipeTiles / 2; ++cp)
    if (2 * cp < np)
      repack_pair<THR>(acc[2 * cp], acc[2 * cp + 1], h1, kw1, cp, lane, TB1, FW1);
  if (nt1 > kPipeTiles)  // wider first layers: the remaining columns from the packed rows
    chain_layer<true, THR>(h0, kw0, W1, N1, 32 * kPipeTiles, h1, TB1, FW1, nullptr, nullptr,
                           row0, M, lane);
  __builtin_amdgcn_wave_barrier();  // h1: this wave's rows only
  chain_layer<true, THR>(h1, kw1, W2, N2, 0, h2, TB2, FW2, nullptr, nullptr, row0, M, lane);
  __builtin_amdgcn_wave_barrier();  // h2: this wave's rows only
  chain_layer<false, false>(h2, kw2, W3, N3, 0, nullptr, nullptr, nullptr, alpha ? AL : nullptr,
                            y, row0, M, lane);
}

template <int DT>
hipError_t launch_dt(const void *x, int64_t ldx, const uint64_t *w1, const uint64_t *w2,
                     const uint64_t *w3, const float *alpha, float *y, int64_t M, int64_t K0,
                     int64_t N1, int64_t N2, int64_t N3, const Chain3Repack &rp, hipStream_t s) {
  const int64_t esize = DT == 0 ? 4 : 2;
  const bool vec = ((uintptr_t)x % 16 == 0) && ((ldx * esize) % 16 == 0 || M == 1);
  const unsigned blocks = (unsigned)((M + 4 * kRows - 1) / (4 * kRows));
  const size_t shmem = (size_t)chain3_lds_words(K0, N1, N2, N3) * sizeof(uint64_t);
  const bool thr = rp.thr1 || rp.flip1 || rp.thr2 || rp.flip2;
#define BNN_CHAIN_LAUNCH(V, T)                                                                 \
  hipLaunchKernelGGL((chain3_kernel<DT, V, T>), dim3(blocks), dim3(256), shmem, s, x, ldx, w1, \
                     w2, w3, alpha, y, (int)M, (int)K0, (int)N1, (int)N2, (int)N3, rp)
  if (vec && thr)
    BNN_CHAIN_LAUNCH(true, true);
  else if (vec)
    BNN_CHAIN_LAUNCH(true, false);
  else if (thr)
    BNN_CHAIN_LAUNCH(false, true);
  else
    BNN_CHAIN_LAUNCH(false, false);
#undef BNN_CHAIN_LAUNCH
  return hipGetLastError();
}

}  // namespace

bool chain3_dims_ok(int64_t K0, int64_t N1, int64_t N2, int64_t N3) {
  auto hidden_ok = [](int64_t d) { return d >= 128 && d <= 64 * kMaxW && d % 128 == 0; };
  return hidden_ok(K0) && hidden_ok(N1) && hidden_ok(N2) && N3 >= 32 && N3 <= 512 &&
         N3 % 32 == 0 && chain3_lds_words(K0, N1, N2, N3) * 8 <= kChain3MaxLds;
}

hipError_t launch_chain3(const void *x, int dtype, int64_t ldx, const uint64_t *w1,
                         const uint64_t *w2, const uint64_t *w3, const float *alpha, float *y,
                         int64_t M, int64_t K0, int64_t N1, int64_t N2, int64_t N3,
                         const Chain3Repack &rp, hipStream_t s) {
  return dtype == 0 ? launch_dt<0>(x, ldx, w1, w2, w3, alpha, y, M, K0, N1, N2, N3, rp, s)
                    : launch_dt<1>(x, ldx, w1, w2, w3, alpha, y, M, K0, N1, N2, N3, rp, s);
}

}  // namespace bnn
