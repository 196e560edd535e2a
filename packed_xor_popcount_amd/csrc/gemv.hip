// gemv.hip -- weight-streaming XOR + popcount product for small M (batch-1
// decode and similar), with an optional fused activation packer.
//
// Same result as the tiled GEMM: <x_m, w_n> = K - 2 * popcount(x_m XOR w_n)
// over the K logical bits ("Binary Math Effectiveness -- why / how / when",
// section 1).  Sections 2.2-2.3 of that page observe that a batch-1 product
// is bound by the bytes of the weights it streams, 1/32 of fp32 once packed;
// this kernel is built to stream the packed W once, at HBM rate.
//
// Design for gfx950 (HBM-bound):
//  * L lanes (a power of two, 4..64) share one column n = one row of W;
//    each lane reads VEC consecutive words (16 B when VEC = 2) per step, so a
//    wave reads G = 64/L whole W rows with fully coalesced loads, and the
//    next step's W words are loaded before the current step's popcounts.
//  * block = 4 wavefronts; one block step covers CB = 4 * G * P columns
//    (P = 1 for latency-bound sizes, 4 when streaming large W, 64 / (4G)
//    for repack); a persistent grid of at most 8 blocks per CU strides over
//    the steps.  Up to 8 activation rows share every W word loaded (rows
//    beyond 8 re-stream W).
//  * XT = 0 reads packed activation words from global memory.  XT = 1 / 2
//    take real-valued fp32 / bf16 activation rows and pack them inside the
//    kernel: each block sign-packs its K-chunk of the (at most 8) rows into
//    LDS, eight lanes per word as the stand-alone packer does, after the
//    first W loads and the alpha loads are already in flight.  A batch-1
//    step is then one launch.
//  * partial counts are summed across the L lanes with xor-shuffles, the
//    column totals are gathered in LDS, and the epilogue stores them
//    coalesced (int32 / alpha-scaled fp32) or ballots 64 of them into one
//    repacked word (P is chosen so that a block step covers 64 columns).
//  * the last word of K is masked (pad bits never count).
#include "../../include/bnn.h"
#include "bnn_internal.h"
#include "sign_bits.h"

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

namespace bnn {
namespace {

constexpr int kMR = 8;            // activation rows sharing one pass over W
constexpr int kChunkWords = 512;  // fused packer: K-chunk held in LDS per row
#ifndef BNN_GEMV_BLOCKS_PER_CU
#define BNN_GEMV_BLOCKS_PER_CU 8
#endif
#ifndef BNN_GEMV_SMALL_P
#define BNN_GEMV_SMALL_P 1
#endif
#ifndef BNN_GEMV_LARGE_P
#define BNN_GEMV_LARGE_P 4  // passes per block step when streaming large W
#endif
constexpr int kBlocksPerCU = BNN_GEMV_BLOCKS_PER_CU;  // persistent grid size (x 256 CUs)

template <int EPI, int L, int VEC, int P, int XT>
__global__ void __launch_bounds__(256)
    gemv_kernel(const void *__restrict__ xv, int64_t ldx, const uint64_t *__restrict__ wp,
                const EpiParams ep, void *__restrict__ yv, int M, int N, int K, int kw, int kcw,
                int xvec) {
  constexpr int G = 64 / L;      // columns per wave per pass
  constexpr int CB = 4 * G * P;  // columns per block step
  static_assert(!is_repack(EPI) || CB == 64, "a repack step covers 64 columns");
  static_assert(256 % CB == 0, "a thread's epilogue column is fixed");
  __shared__ uint32_t res[kMR][CB];
  extern __shared__ __attribute__((aligned(16))) uint64_t xs[];  // XT != 0: [rows][kcw]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane / L;
  const int part = lane % L;
  const uint64_t tmask = tail_mask(K);
  const int nw = (N + 63) >> 6;
  const int nsteps = (N + CB - 1) / CB;
  const uint64_t *xp = static_cast<const uint64_t *>(xv);

  // Sign-pack activation rows mb .. mb+mrows-1, words c0 .. c0+cw-1 into LDS
  // (eight lanes per word, as the stand-alone packer does; each lane group
  // builds up to kS words per round with all their loads in flight).  The
  // load and finish halves of a round are separate so that the first round
  // can be loaded before the W stream starts and finished after it.
  constexpr int kS = 4;
  constexpr int DTX = XT == 2 ? 1 : 0;
  auto pack_load = [&](int mb, int mrows, int c0, int cw, int q0, Raw8(&raw)[kS]) {
    const int grp = tid >> 3, t = tid & 7;
    const int total = mrows * cw;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const int q = q0 + s * 32 + grp;
      int n_ok = 0;
      int64_t e0 = 0;
      if (q < total) {
        const int r = q / cw, w = q - r * cw;
        const int64_t e = (int64_t)(c0 + w) * 64 + 8 * t;
        const int64_t left = (int64_t)K - e;
        n_ok = left >= 8 ? 8 : (left > 0 ? (int)left : 0);
        e0 = (int64_t)(mb + r) * ldx + e;
      }
      if (xvec)
        raw[s] = load_raw8<DTX, true>(xv, e0, n_ok);
      else
        raw[s] = load_raw8<DTX, false>(xv, e0, n_ok);
    }
  };
  auto pack_finish = [&](int mrows, int cw, int q0, const Raw8(&raw)[kS]) {
    const int grp = tid >> 3, t = tid & 7;
    const int total = mrows * cw;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const int q = q0 + s * 32 + grp;
      const uint64_t word = word_from_bytes(byte_of<DTX>(raw[s]), t);
      if (t == 0 && q < total) {
        const int r = q / cw, w = q - r * cw;
        xs[r * kcw + w] = word;
      }
    }
  };
  auto pack_x = [&](int mb, int mrows, int c0, int cw) {
    for (int q0 = 0; q0 < mrows * cw; q0 += 32 * kS) {  // uniform trip count
      Raw8 raw[kS];
      pack_load(mb, mrows, c0, cw, q0, raw);
      pack_finish(mrows, cw, q0, raw);
    }
  };
  // With at most 8 rows and one K-chunk, the packed activations stay in LDS
  // for every column step of this block: they are packed once, right after
  // the first step's W loads are issued (so the two latencies overlap).
  const bool x_once = XT != 0 && M <= kMR && kw <= kcw;
  bool x_ready = false;

  for (int step = blockIdx.x; step < nsteps; step += gridDim.x) {
    const int64_t nb = (int64_t)step * CB;
    // W and alpha are read from clamped, always in-bounds addresses: the loads
    // are unconditional (no zero-initialised destination registers for the
    // compiler to guard with waits), W first; lanes whose unit is past the
    // chunk skip the popcounts and columns past N are never stored.
    uint64_t wa[P][VEC], wb[P][VEC];
    float a_pre = 0.0f;
    // Threshold of column nb + lane and flip word of this step's 64 columns
    // (threshold repack; loaded here so that K = 0 has them too).
    int32_t t_pre = 0;
    uint64_t f_pre = 0;
    if (EPI == kEpiRepackThr) {
      t_pre = thr_of(ep, nb + lane, N);
      f_pre = flip_of(ep, nb >> 6, N);
    }

    for (int mb = 0; mb < M; mb += kMR) {
      const int mrows = (M - mb) < kMR ? (M - mb) : kMR;
      uint32_t acc[P][kMR];
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int r = 0; r < kMR; ++r) acc[p][r] = 0;

      for (int c0 = 0; c0 < kw; c0 += kcw) {
        const int cw = (kw - c0) < kcw ? (kw - c0) : kcw;
        const int ubeg = c0 / VEC, uend = (c0 + cw) / VEC;  // uend > ubeg

        auto load_w = [&](int ub, uint64_t(&w)[P][VEC]) {
          int u = ub + part;
          u = u < uend ? u : uend - 1;
#pragma unroll
          for (int p = 0; p < P; ++p) {
            int64_t n = nb + (int64_t)(p * 4 + wave) * G + sub;
            n = n < N ? n : N - 1;
            const uint64_t *src = wp + n * kw + (int64_t)u * VEC;
            if (VEC == 2) {
              const ulonglong2 t = *reinterpret_cast<const ulonglong2 *>(src);
              w[p][0] = t.x;
              w[p][VEC - 1] = t.y;
            } else {
              w[p][0] = src[0];
            }
          }
        };
        load_w(ubeg, wa);
        if (EPI == BNN_EPI_SCALED) {
          // The epilogue column of this thread is fixed (CB divides 256).
          int64_t n = nb + (tid % CB);
          n = n < N ? n : N - 1;
          a_pre = ep.alpha[n];
        }

        if constexpr (XT != 0) {
          if (x_once) {
            if (!x_ready) {  // uniform
              pack_x(0, M, 0, kw);
              __syncthreads();
              x_ready = true;
            }
          } else {
            __syncthreads();  // the previous chunk's words are consumed
            pack_x(mb, mrows, c0, cw);
            __syncthreads();
          }
        }

        for (int ub = ubeg; ub < uend; ub += L) {
          if (ub + L < uend) load_w(ub + L, wb);
          const int u = ub + part;
          if (u < uend) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              const int word = u * VEC + v;
              const uint64_t wm = (word == kw - 1) ? tmask : ~uint64_t(0);
#pragma unroll
              for (int r = 0; r < kMR; ++r) {
                if (r >= mrows) break;
                uint64_t x;
                if constexpr (XT == 0)
                  x = xp[(int64_t)(mb + r) * kw + word] & wm;
                else
                  x = xs[r * kcw + (word - c0)] & wm;
#pragma unroll
                for (int p = 0; p < P; ++p) {
                  const uint64_t d = x ^ (wa[p][v] & wm);
                  acc[p][r] = popc_acc((uint32_t)(d >> 32), popc_acc((uint32_t)d, acc[p][r]));
                }
              }
            }
          }
#pragma unroll
          for (int p = 0; p < P; ++p)
#pragma unroll
            for (int v = 0; v < VEC; ++v) wa[p][v] = wb[p][v];
        }
      }

      // Sum the L partial counts of each column (all lanes of a group end with the total).
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int r = 0; r < kMR; ++r) {
          if (r >= mrows) break;
          uint32_t a = acc[p][r];
#pragma unroll
          for (int off = L / 2; off >= 1; off >>= 1) a += __shfl_xor(a, off, 64);
          acc[p][r] = a;
        }
      __syncthreads();  // res is free (the previous epilogue has read it)
      if (part == 0) {
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int r = 0; r < kMR; ++r) {
            if (r >= mrows) break;
            res[r][(p * 4 + wave) * G + sub] = acc[p][r];
          }
      }
      __syncthreads();

      if (is_repack(EPI)) {
        if (wave == 0) {
          const int64_t n = nb + lane;
          for (int r = 0; r < mrows; ++r) {
            const int dot = (int)((uint32_t)K - 2u * res[r][lane]);
            const uint64_t word = __builtin_amdgcn_ballot_w64(n < N && dot <= t_pre) ^ f_pre;
            if (lane == 0) static_cast<uint64_t *>(yv)[(int64_t)(mb + r) * nw + (nb >> 6)] = word;
          }
        }
      } else {
        const int c = tid % CB;
        const int64_t n = nb + c;
        if (n < N) {
          for (int r = tid / CB; r < mrows; r += 256 / CB) {
            const int dot = (int)((uint32_t)K - 2u * res[r][c]);
            const int64_t o = (int64_t)(mb + r) * N + n;
            if (EPI == BNN_EPI_I32)
              static_cast<int32_t *>(yv)[o] = dot;
            else
              static_cast<float *>(yv)[o] = __fmul_rn((float)dot, a_pre);
          }
        }
      }
    }
  }
}

// Batch decode form (M <= 8): every lane holds at most one unit (VEC words)
// of each W row it serves (units <= L), so a block step is one
// straight-line round: issue the scale loads, the activation loads (first
// step of the block only), then the W loads; popcounts; reduction;
// epilogue.  The same arithmetic and epilogues as gemv_kernel.  XT 1 / 2:
// activation rows given as real fp32 / bf16 values (K a multiple of 64,
// rows 16-byte aligned), packed into LDS while the first W words are in
// flight.  XT 0: packed activation rows (the named products at small M);
// a lane's activation words are the same for every step, so they are
// loaded into registers once.  TAIL (XT 0 only): K is not a multiple of 64
// and the last word's pad bits are masked.
template <int EPI, int L, int VEC, int P, int XT, bool TAIL>
__global__ void __launch_bounds__(256)
    gemv_act_kernel(const void *__restrict__ xv, int64_t ldx, const uint64_t *__restrict__ wp,
                    const EpiParams ep, void *__restrict__ yv, int M, int N, int K, int kw) {
  constexpr int DT = XT == 2 ? 1 : 0;
  static_assert(!TAIL || XT == 0, "real-valued rows hold whole words");
  constexpr int G = 64 / L;
  constexpr int CB = 4 * G * P;
  constexpr int kS = 4;  // activation words per lane group per round
  static_assert(!is_repack(EPI) || CB == 64, "a repack step covers 64 columns");
  __shared__ uint32_t res[kMR][CB];
  extern __shared__ __attribute__((aligned(16))) uint64_t xs[];  // [M][kw]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane / L;
  const int part = lane % L;
  const int grp = tid >> 3, t8 = tid & 7;
  const int nw = (N + 63) >> 6;
  const int nsteps = (N + CB - 1) / CB;
  const int units = kw / VEC;   // >= 1 (K > 0 here)
  const bool u_ok = part < units;
  const int u = u_ok ? part : units - 1;
  const int total = M * kw;     // activation words to pack

  // XT 0: this lane's activation words (unit u of every row), masked past
  // K in the last word, loaded once.
  uint64_t xw[kMR][VEC];
  if constexpr (XT == 0) {
    const uint64_t *xp = static_cast<const uint64_t *>(xv);
#pragma unroll
    for (int rr = 0; rr < kMR; ++rr) {
      if (rr >= M) break;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const int word = u * VEC + v;
        uint64_t x = xp[(int64_t)rr * ldx + word];
        if (TAIL && word == kw - 1) x &= tail_mask(K);
        xw[rr][v] = x;
      }
    }
  }
  // Pad-bit mask of this lane's words (TAIL): W's pad bits must not count.
  uint64_t wmask[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) wmask[v] = (TAIL && u * VEC + v == kw - 1) ? tail_mask(K) : ~0ull;

  // Every activation row holds whole 16-byte-aligned groups of 8 elements
  // (the launcher checks this), so the loads are unconditional vector loads;
  // slots past the last word re-read the last one and are not stored.
  // Rounds s past the last word are skipped (uniform branches); with a
  // single row the word index needs no division.
  auto x_round = [&](int q0, Raw8(&raw)[kS]) {
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      if (q0 + s * 32 >= total) break;
      int q = q0 + s * 32 + grp;
      q = q < total ? q : total - 1;
      int64_t e0;
      if (M == 1) {
        e0 = (int64_t)q * 64 + 8 * t8;
      } else {
        const int r = q / kw, wd = q - r * kw;
        e0 = (int64_t)r * ldx + (int64_t)wd * 64 + 8 * t8;
      }
      raw[s] = load_raw8<DT, true>(xv, e0, 8);
    }
  };
  auto x_store = [&](int q0, const Raw8(&raw)[kS]) {
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      if (q0 + s * 32 >= total) break;
      const int q = q0 + s * 32 + grp;
      const uint64_t word = word_from_bytes(byte_of<DT>(raw[s]), t8);
      if (t8 == 0 && q < total) xs[q] = word;  // row r, word w at r * kw + w == q
    }
  };

  // Operands of one block step, loaded before they are used: the scales (or
  // threshold and flip word) of the columns this lane stores and this lane's
  // W unit of each pass.  W and the scales come from clamped, always
  // in-bounds addresses, so the loads are unconditional.
  struct StepRegs {
    float a[P];
    int32_t t;
    uint64_t f;
    uint64_t w[P][VEC];
  };
  auto load_step = [&](int step, StepRegs &r) {
    const int64_t nb = (int64_t)step * CB;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      r.a[p] = 0.0f;
      if (EPI == BNN_EPI_SCALED) {
        int64_t n = nb + (int64_t)(p * 4 + wave) * G + sub;
        n = n < N ? n : N - 1;
        r.a[p] = ep.alpha[n];
      }
    }
    r.t = 0;
    r.f = 0;
    if (EPI == kEpiRepackThr) {  // repack is stored by wave 0, one column per lane
      r.t = thr_of(ep, nb + lane, N);
      r.f = flip_of(ep, nb >> 6, N);
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      int64_t n = nb + (int64_t)(p * 4 + wave) * G + sub;
      n = n < N ? n : N - 1;
      const uint64_t *src = wp + n * kw + (int64_t)u * VEC;
      // W is read once per call: non-temporal loads keep it from
      // displacing the activation row and the scales in the caches
      // (batch-1 4096 x 4096: 3.01 -> 2.41 us per step).
      if (VEC == 2) {
        const u64x2 v = __builtin_nontemporal_load(reinterpret_cast<const u64x2 *>(src));
        r.w[p][0] = v.x;
        r.w[p][VEC - 1] = v.y;
      } else {
        r.w[p][0] = __builtin_nontemporal_load(src);
      }
    }
  };
  auto run_step = [&](int step, const StepRegs &r) {
    const int64_t nb = (int64_t)step * CB;
    uint32_t acc[P][kMR];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int rr = 0; rr < kMR; ++rr) acc[p][rr] = 0;
    if (u_ok) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const int word = u * VEC + v;
#pragma unroll
        for (int rr = 0; rr < kMR; ++rr) {
          if (rr >= M) break;
          uint64_t x;
          if constexpr (XT == 0)
            x = xw[rr][v];
          else
            x = xs[rr * kw + word];
#pragma unroll
          for (int p = 0; p < P; ++p) {
            uint64_t d = x ^ r.w[p][v];
            if (TAIL) d &= wmask[v];
            acc[p][rr] = popc_acc((uint32_t)(d >> 32), popc_acc((uint32_t)d, acc[p][rr]));
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int rr = 0; rr < kMR; ++rr) {
        if (rr >= M) break;
        acc[p][rr] = group_sum<L>(acc[p][rr]);
      }

    if (is_repack(EPI)) {
      __syncthreads();  // res is free (the previous step's epilogue has read it)
      if (part == 0) {
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int rr = 0; rr < kMR; ++rr) {
            if (rr >= M) break;
            res[rr][(p * 4 + wave) * G + sub] = acc[p][rr];
          }
      }
      __syncthreads();
      if (wave == 0) {
        const int64_t n = nb + lane;
        for (int rr = 0; rr < M; ++rr) {
          const int dot = (int)((uint32_t)K - 2u * res[rr][lane]);
          const uint64_t word = __builtin_amdgcn_ballot_w64(n < N && dot <= r.t) ^ r.f;
          if (lane == 0) static_cast<uint64_t *>(yv)[(int64_t)rr * nw + (nb >> 6)] = word;
        }
      }
    } else if (part == 0) {
      // Every lane of a group holds its column's total: the first one stores.
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int64_t n = nb + (int64_t)(p * 4 + wave) * G + sub;
        if (n >= N) continue;
#pragma unroll
        for (int rr = 0; rr < kMR; ++rr) {
          if (rr >= M) break;
          const int dot = (int)((uint32_t)K - 2u * acc[p][rr]);
          const int64_t o = (int64_t)rr * N + n;
          if (EPI == BNN_EPI_I32)
            static_cast<int32_t *>(yv)[o] = dot;
          else
            static_cast<float *>(yv)[o] = __fmul_rn((float)dot, r.a[p]);
        }
      }
    }
  };

  // First step: the activation loads go out ahead of the W loads, so the
  // packing that must follow them overlaps the W latency.  Later steps run
  // in pairs whose operands are loaded one step ahead (blocks with several
  // steps stream W continuously); a pair's second half exists only when the
  // block has that step, so single-step blocks load nothing extra.  The two
  // register sets are never copied (a copy would wait for its load).
  StepRegs ra;
  if constexpr (XT != 0) {
    Raw8 raw[kS];
    x_round(0, raw);
    load_step(blockIdx.x, ra);
    x_store(0, raw);
    for (int q0 = 32 * kS; q0 < total; q0 += 32 * kS) {
      x_round(q0, raw);
      x_store(q0, raw);
    }
    __syncthreads();
  } else {
    load_step(blockIdx.x, ra);
    // the activation words are settled once, behind the first W loads
#pragma unroll
    for (int rr = 0; rr < kMR; ++rr) {
      if (rr >= M) break;
#pragma unroll
      for (int v = 0; v < VEC; ++v) xw[rr][v] = settled(xw[rr][v]);
    }
  }
  // A block with one step (the batch-1 sizes) runs it and ends.  Otherwise
  // the prefetches are unconditional -- past the block's last step they
  // re-read its current step -- so that the compiler's count of loads in
  // flight is exact and each step waits for its own loads only.
  if (blockIdx.x + gridDim.x >= nsteps) {
    run_step(blockIdx.x, ra);
    return;
  }
  for (int step = blockIdx.x; step < nsteps; step += 2 * gridDim.x) {
    const int sb = step + gridDim.x, sa = step + 2 * gridDim.x;
    StepRegs rb;
    load_step(sb < nsteps ? sb : step, rb);
    run_step(step, ra);
    load_step(sa < nsteps ? sa : step, ra);
    if (sb < nsteps) run_step(sb, rb);  // uniform
  }
}

struct Args {
  const void *x;
  int64_t ldx;
  const uint64_t *wp;
  EpiParams ep;
  void *y;
  int M, N, K, kw, kcw, xvec;
};

template <int EPI, int L, int VEC, int XT, int P>
hipError_t launch_lp(const Args &a, hipStream_t s) {
  constexpr int CB = 4 * (64 / L) * P;
  const int64_t steps = ((int64_t)a.N + CB - 1) / CB;
  // Persistent grid: at most kBlocksPerCU blocks per CU, striding over
  // column steps (so the fused packer runs once per block).
  const int64_t cap = 256 * kBlocksPerCU;
  const int64_t blocks = steps < cap ? steps : cap;
  const int rows = a.M < kMR ? a.M : kMR;
  // Batch decode form: at most 8 rows and at most one unit per lane; real
  // rows hold whole 16-byte-aligned words, packed rows may end in a partial
  // word.
  if (a.M <= kMR && a.kw > 0 && a.kw / VEC <= L) {
    if constexpr (XT != 0) {
      if (a.K % 64 == 0 && a.xvec) {
        const size_t shmem = (size_t)a.M * a.kw * sizeof(uint64_t);
        hipLaunchKernelGGL((gemv_act_kernel<EPI, L, VEC, P, XT, false>), dim3((unsigned)blocks),
                           dim3(256), shmem, s, a.x, a.ldx, a.wp, a.ep, a.y, a.M, a.N, a.K,
                           a.kw);
        return hipGetLastError();
      }
    } else {
      if (a.K % 64 == 0)
        hipLaunchKernelGGL((gemv_act_kernel<EPI, L, VEC, P, 0, false>), dim3((unsigned)blocks),
                           dim3(256), 0, s, a.x, a.ldx, a.wp, a.ep, a.y, a.M, a.N, a.K, a.kw);
      else
        hipLaunchKernelGGL((gemv_act_kernel<EPI, L, VEC, P, 0, true>), dim3((unsigned)blocks),
                           dim3(256), 0, s, a.x, a.ldx, a.wp, a.ep, a.y, a.M, a.N, a.K, a.kw);
      return hipGetLastError();
    }
  }
  const size_t shmem = XT == 0 ? 0 : (size_t)rows * a.kcw * sizeof(uint64_t);
  hipLaunchKernelGGL((gemv_kernel<EPI, L, VEC, P, XT>), dim3((unsigned)blocks), dim3(256), shmem,
                     s, a.x, a.ldx, a.wp, a.ep, a.y, a.M, a.N, a.K, a.kw, a.kcw, a.xvec);
  return hipGetLastError();
}

template <int EPI, int L, int VEC, int XT>
hipError_t launch_l(const Args &a, hipStream_t s) {
  if constexpr (is_repack(EPI)) {
    return launch_lp<EPI, L, VEC, XT, L / 4>(a, s);  // a step covers 64 columns
  } else {
    // One pass per step while one wave of blocks covers N (latency-bound
    // sizes: more, smaller blocks); four passes beyond that, so each lane
    // keeps four W loads in flight per step when streaming large W.
    constexpr int CB1 = 4 * (64 / L);
    if ((int64_t)a.N <= (int64_t)CB1 * 256 * kBlocksPerCU)
      return launch_lp<EPI, L, VEC, XT, BNN_GEMV_SMALL_P>(a, s);
    return launch_lp<EPI, L, VEC, XT, BNN_GEMV_LARGE_P>(a, s);
  }
}

template <int EPI, int VEC, int XT>
hipError_t launch_vec(const Args &a, hipStream_t s) {
  const int units = a.kw / VEC;
  if (units <= 4) return launch_l<EPI, 4, VEC, XT>(a, s);
  if (units <= 8) return launch_l<EPI, 8, VEC, XT>(a, s);
  if (units <= 16) return launch_l<EPI, 16, VEC, XT>(a, s);
  if (units <= 32) return launch_l<EPI, 32, VEC, XT>(a, s);
  return launch_l<EPI, 64, VEC, XT>(a, s);
}

template <int EPI, int XT>
hipError_t launch_epi(const Args &a, hipStream_t s) {
  const bool x16 = XT != 0 || ((uintptr_t)a.x % 16 == 0);
  const bool vec2 = (a.kw % 2 == 0) && x16 && ((uintptr_t)a.wp % 16 == 0);
  if (vec2) return launch_vec<EPI, 2, XT>(a, s);
  return launch_vec<EPI, 1, XT>(a, s);
}

template <int XT>
hipError_t launch_xt(const Args &a, int epilogue, hipStream_t s) {
  switch (epilogue) {
    case BNN_EPI_I32: return launch_epi<BNN_EPI_I32, XT>(a, s);
    case BNN_EPI_SCALED: return launch_epi<BNN_EPI_SCALED, XT>(a, s);
    case kEpiRepackThr: return launch_epi<kEpiRepackThr, XT>(a, s);
    default: return launch_epi<BNN_EPI_REPACK, XT>(a, s);
  }
}

}  // namespace

hipError_t launch_gemv(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y,
                       int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s) {
  const int kw = (int)((K + 63) / 64);
  const Args a{xp, kw, wp, ep, y, (int)M, (int)N, (int)K, kw, kw > 0 ? kw : 1, 0};
  return launch_xt<0>(a, epilogue, s);
}

hipError_t launch_gemv_act(const void *x, int dtype, int64_t ldx, const uint64_t *wp,
                           const EpiParams &ep, void *y, int64_t M, int64_t N, int64_t K,
                           int epilogue, hipStream_t s) {
  const int kw = (int)((K + 63) / 64);
  const int64_t esize = dtype == 0 ? 4 : 2;
  // 16-byte activation loads need every row start 16-byte aligned.
  const int xvec = ((uintptr_t)x % 16 == 0) && ((ldx * esize) % 16 == 0 || M == 1);
  // K-chunk per row in LDS: even (for 16-byte W loads), at most kChunkWords.
  int kcw = kw < kChunkWords ? kw : kChunkWords;
  if (kcw < 1) kcw = 1;
  const Args a{x, ldx, wp, ep, y, (int)M, (int)N, (int)K, kw, kcw, xvec};
  return dtype == 0 ? launch_xt<1>(a, epilogue, s) : launch_xt<2>(a, epilogue, s);
}

}  // namespace bnn
