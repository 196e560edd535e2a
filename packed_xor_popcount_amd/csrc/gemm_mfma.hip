// gemm_mfma.hip -- packed binary GEMM on the gfx950 matrix cores (large M).
//
// The result is the same integer as the XOR + popcount kernels:
// <x_m, w_n> = K - 2 * popcount(x_m XOR w_n) = sum_k x[k] * w[k] over the K
// logical elements, x, w in {+1, -1} ("Binary Math Effectiveness -- why /
// how / when", section 1: the identity is exact, so the plain sum of
// products is the same number).  Section 3 of that page notes that dense
// tensor units usually beat naive bit kernels; on MI355X the FP4 matrix
// rate is about 8x the VALU XOR + popcount issue rate, so for large M the
// sum of products is taken on the matrix cores instead:
//
//  * a packed bit b is an FP4 (e2m1) operand value (+1.0 = 0x2 when b = 0,
//    -1.0 = 0xA when b = 1): the packed bit IS the FP4 sign bit, so no table
//    is needed.  A 32-bit chunk x of a packed row becomes the four operand
//    registers ((x << (3 - r)) & 0x88888888) | 0x22222222, r = 0..3, i.e.
//    register r nibble j holds bit 4j + r.  This permutes the K elements
//    inside the chunk; a dot product does not depend on the order of its
//    terms, and A and B are unpacked by the same rule, so the product is
//    unchanged.  Seven VALU ops unpack 32 elements.
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP4 and unit
//    scales (E8M0 127) accumulates in fp32.  Each product is +-1 (or 0 for a
//    masked pad element), so every partial sum is an integer of magnitude
//    <= K and is exact while K <= 2^24 (the library uses this kernel only
//    then).  The final fp32 accumulator IS the integer dot.
//  * pad elements (k >= K) get zero nibbles in the A operand, so they add
//    nothing whatever the pad bits of either operand hold.
//
// Work split.  A block is 4 waves arranged WR x WC; a wave owns RB x CB
// tiles of 32 x 32 outputs.  The unpack costs 5.5 VALU ops per operand
// register set (the two 32-element halves of a word share their 64-bit
// shifts) and one set feeds CB (A) or RB (B) MFMAs of 32 cycles, so VALU
// per MFMA = 5.5 (RB + CB) / (RB CB): 2.75 at 4 x 4 tiles.  The large
// configuration is therefore 2 x 2 waves of 4 x 4 tiles (block tile
// 256 x 256, one wave per SIMD, accumulators in the AGPRs); small shapes use
// 4 x 1 waves of 1 x 2 or 2 x 2.
//
// K loop.  A step is SW words (64 SW elements of K): lanes 0-31 hold the
// first SW / 2 words of the step of their row / column, lanes 32-63 the
// last SW / 2; slice (i, q) pairs half q of word i of both lane halves.  The
// words are read with buffer loads through per-block resources: each
// lane's row offset is fixed and the step offset is a scalar, so a step
// costs no vector address arithmetic, and every load outside the block's
// rows returns 0 (no load can leave the matrices).  Two register sets
// ping-pong: step s+1 is in flight while step s runs.  Inside a step, slice
// j+1 is unpacked while slice j's MFMAs run.
//
// Tile order.  Hardware places block b on XCD b % 8; block b takes logical
// tile (b % 8) * (T / 8) + b / 8 (T tiles, column-tile major), so each
// XCD's L2 holds all of X but only an eighth of W.
//
// Output layout of a 32 x 32 tile (lane l, accumulator register v): column
// l % 32, row 8 (v / 4) + 4 (l / 32) + v % 4.  The repack epilogue ballots
// two neighbouring tiles: the low 32 ballot bits are one row's 32 columns,
// the high 32 bits those of the row 4 below.
#include "../../include/bnn.h"
#include "bnn_internal.h"
#include "fp4_ops.h"

namespace bnn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


typedef int v4i __attribute__((ext_vector_type(4)));

// Operand registers (the four used nibble registers of an FP4 operand) of
// the 32-bit chunk c: register r = ((c << (3 - r)) & 0x88888888) | 0x22222222.
__device__ __forceinline__ v4i fp4_chunk(uint32_t c, uint32_t c8, uint32_t c2) {
  v4i o;
  o[0] = (int)and_or(c << 3, c8, c2);
  o[1] = (int)and_or(c << 2, c8, c2);
  o[2] = (int)and_or(c << 1, c8, c2);
  o[3] = (int)and_or(c, c8, c2);
  return o;
}

// The eight-register operand of the FP4 MFMA: an FP4 operand uses the first
// four registers only.
__device__ __forceinline__ v8i fp4_operand(v4i o) {
  const v4i z = {0, 0, 0, 0};
  return __builtin_shufflevector(o, z, 0, 1, 2, 3, 4, 5, 6, 7);
}

// mask_operand on the four used registers.
__device__ __forceinline__ v4i mask4(v4i a, uint32_t valid) {
  const v8i m = mask_operand(fp4_operand(a), valid);
  return (v4i){m[0], m[1], m[2], m[3]};
}

// Epilogue operands of the columns nc[cb] + li (li = lane % 32): the scale,
// or the threshold as an fp32 bound that is exact against the (exact, |d| <=
// K <= 2^24) accumulators -- +inf / -inf outside [-K, K] -- and the flip word
// of each 64-column pair (nc[2cp], nc[2cp] + 32).  Loaded before the K loop.
template <int EPI, int CB>
__device__ __forceinline__ void epilogue_operands(const EpiParams &ep, const int (&nc)[CB], int li,
                                                  int N, int K, float (&a_pre)[CB],
                                                  uint64_t (&f_pre)[CB / 2 > 0 ? CB / 2 : 1]) {
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = nc[cb] + li;
    a_pre[cb] = (EPI == BNN_EPI_SCALED && n < N) ? ep.alpha[n < N ? n : N - 1] : 0.0f;
    if (EPI == kEpiRepackThr) {
      const int32_t t = thr_of(ep, n, N);
      a_pre[cb] = t >= K ? __builtin_inff() : (t < -K ? -__builtin_inff() : (float)t);
    }
  }
#pragma unroll
  for (int cp = 0; cp < (CB / 2 > 0 ? CB / 2 : 1); ++cp)
    f_pre[cp] = (EPI == kEpiRepackThr && CB >= 2) ? flip_of(ep, nc[2 * cp] >> 6, N) : 0;
}

// Stores of RB x CB accumulator tiles: acc[rb][cb][v] is the exact integer
// dot of row mr[rb] + 8 (v / 4) + 4h + v % 4 and column nc[cb] + li
// (h = lane / 32, li = lane % 32); column pairs (2cp, 2cp + 1) are 64
// consecutive columns starting at a multiple of 64.  Every load has been
// waited for before this (so that no store waits).
template <int EPI, int RB, int CB>
__device__ __forceinline__ void store_tiles(const v16f (&acc)[RB][CB], const float (&a_pre)[CB],
                                            const uint64_t (&f_pre)[CB / 2 > 0 ? CB / 2 : 1],
                                            const int (&mr)[RB], const int (&nc)[CB], int h,
                                            int li, void *__restrict__ yv, int M, int N) {
  if (is_repack(EPI)) {
    const int nw = (N + 63) >> 6;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cp = 0; cp < CB / 2; ++cp) {
        const int na = nc[2 * cp] + li, nb2 = na + 32;
        const int wi = nc[2 * cp] >> 6;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // bit set (-1) where the dot is <= the threshold (0 for the plain repack)
          const uint64_t lo = __builtin_amdgcn_ballot_w64(na < N && acc[rb][2 * cp][v] <= a_pre[2 * cp]);
          const uint64_t hi =
              __builtin_amdgcn_ballot_w64(nb2 < N && acc[rb][2 * cp + 1][v] <= a_pre[2 * cp + 1]);
          // lane 0 writes row r, lane 32 writes row r + 4
          const int r = mr[rb] + 8 * (v >> 2) + (v & 3) + 4 * h;
          const uint64_t word = (h ? ((hi & 0xFFFFFFFF00000000ull) | (lo >> 32))
                                   : ((hi << 32) | (lo & 0xFFFFFFFFull))) ^ f_pre[cp];
          if (li == 0 && r < M && wi < nw) static_cast<uint64_t *>(yv)[(int64_t)r * nw + wi] = word;
        }
      }
  } else {
    // Tiles wholly inside M store their 16 values without a row test
    // (straight-line stores: no branch per value).
    const int64_t ld = N;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int mt = mr[rb] + 4 * h;  // row of v = 0 for this lane
      const bool full_rows = mr[rb] + 32 <= M;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int n = nc[cb] + li;
        if (n >= N) continue;
        const float a = a_pre[cb];
        const int64_t base = (int64_t)mt * ld + n;
        auto put = [&](int v) __attribute__((always_inline)) {
          // (8 (v / 4) + v % 4) * ld is the same for every lane
          const int64_t o = base + (int64_t)(8 * (v >> 2) + (v & 3)) * ld;
          if (EPI == BNN_EPI_I32)
            static_cast<int32_t *>(yv)[o] = (int)acc[rb][cb][v];
          else
            static_cast<float *>(yv)[o] = __fmul_rn(acc[rb][cb][v], a);
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
}

// The K loop of one wave tile: acc[rb][cb] += the sum over K of the
// products of A tile rb (the X rows at aoff[rb] in ares) and B tile cb (the
// W rows at boff[cb] in bres).
template <int RB, int CB, int SW>
__device__ __forceinline__ void k_loop(v16f (&acc)[RB][CB], const __amdgpu_buffer_rsrc_t ares,
                                       const __amdgpu_buffer_rsrc_t bres, const uint32_t (&aoff)[RB],
                                       const uint32_t (&boff)[CB], int K, int kw, int h,
                                       uint32_t c8, uint32_t c2) {
  constexpr int kSW = SW, kHW = SW / 2;  // words per step, per lane
  const int nsteps = (kw + kSW - 1) / kSW;
  const int nclean = (K >> 6) / kSW;  // steps with every element inside K

  // Operand sets: set p < RB is A tile p (rows), set RB + c is B tile c
  // (columns).  Step registers: 32-bit chunks, [set][chunk] with chunk
  // 2i + q = half q of this lane's word i.
  constexpr int NS = RB + CB;
  typedef uint32_t Buf[NS][2 * kHW];
  auto load_step = [&](int s, Buf &u) __attribute__((always_inline)) {
    const int so = s * (kSW * 8);
#pragma unroll
    for (int p = 0; p < NS; ++p)
#pragma unroll
      for (int j = 0; j < kHW / 2; ++j) {
        const u32x4 v = p < RB
                            ? __builtin_amdgcn_raw_buffer_load_b128(ares, aoff[p] + 16 * j, so, 0)
                            : __builtin_amdgcn_raw_buffer_load_b128(bres, boff[p - RB] + 16 * j, so, 0);
        u[p][4 * j + 0] = v.x; u[p][4 * j + 1] = v.y;
        u[p][4 * j + 2] = v.z; u[p][4 * j + 3] = v.w;
      }
  };
  // Slices.  Slice j of a step (j = 2i + q: half q of this lane's word i)
  // unpacks NS operand sets and feeds RB * CB MFMAs.  The slices run as a
  // software pipeline: while the MFMAs of slice j issue, the VALU unpacks
  // slice j + 1 (of the next step after a step's last slice) into the other
  // of two operand register sets.  The two halves of a word share their
  // shifts (as in fp4_operands): the even slice of word i takes the three
  // 64-bit shifts of the word and keeps their high halves, the odd slice
  // only masks those -- 5.5 instead of 7 VALU ops per set.  Each set's
  // unpack is split in two work items, and the 2 NS items are placed
  // between the MFMAs by hand (a scheduling barrier after each group), so
  // that the VALU ops are spread evenly over the matrix-core instructions.
  struct Ops {
    v4i s[NS];
  };
  Ops op0, op1;
  uint32_t keep[NS][3], lows[NS][3];
  // Item k of set p for the even slice 2i.  `next`: a step register set
  // whose loads may still be in flight; its shifts are then volatile, so
  // that the wait for the loads stays here (the scheduler would otherwise
  // pull the shifts up to the loads).
  auto even_item = [&](const Buf &u, int i, Ops &o, bool next, int p, int k) __attribute__((always_inline)) {
    if (k == 0) {
      // the shifts, and the one register that needs none (no shift result
      // is read right after it is written: that would cost a wait state)
      const uint64_t w = ((uint64_t)u[p][2 * i + 1] << 32) | u[p][2 * i];
      const uint64_t s1 = shl64<1>(w, next), s2 = shl64<2>(w, next), s3 = shl64<3>(w, next);
      keep[p][0] = (uint32_t)(s3 >> 32);
      keep[p][1] = (uint32_t)(s2 >> 32);
      keep[p][2] = (uint32_t)(s1 >> 32);
      lows[p][0] = (uint32_t)s3;
      lows[p][1] = (uint32_t)s2;
      lows[p][2] = (uint32_t)s1;
      o.s[p][3] = (int)and_or(u[p][2 * i], c8, c2);
    } else {
      o.s[p][0] = (int)and_or(lows[p][0], c8, c2);
      o.s[p][1] = (int)and_or(lows[p][1], c8, c2);
      o.s[p][2] = (int)and_or(lows[p][2], c8, c2);
    }
  };
  // Item k of set p for the odd slice 2i + 1, from the kept shifts.
  auto odd_item = [&](const Buf &u, int i, Ops &o, int p, int k) __attribute__((always_inline)) {
    if (k == 0) {
      o.s[p][0] = (int)and_or(keep[p][0], c8, c2);
      o.s[p][1] = (int)and_or(keep[p][1], c8, c2);
    } else {
      o.s[p][2] = (int)and_or(keep[p][2], c8, c2);
      o.s[p][3] = (int)and_or(u[p][2 * i + 1], c8, c2);
    }
  };
  auto mfma = [&](const Ops &o, int q) __attribute__((always_inline)) {
    const int rb = q / CB, cb = q % CB;
    acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        fp4_operand(o.s[rb]), fp4_operand(o.s[RB + cb]), acc[rb][cb], kFmtFp4, kFmtFp4, 0,
        kScaleOne, 0, kScaleOne);
  };
  // The MFMAs of slice operands o; after MFMA q, the work items
  // [q W / NM, (q + 1) W / NM) of the next slice (W = 2 NS items, NM MFMAs).
  constexpr int NM = RB * CB, W = 2 * NS;
  auto slice_even_next = [&](const Ops &o, const Buf &u, int i, Ops &d, bool next) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      mfma(o, q);
#pragma unroll
      for (int w = q * W / NM; w < (q + 1) * W / NM; ++w) even_item(u, i, d, next, w >> 1, w & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto slice_odd_next = [&](const Ops &o, const Buf &u, int i, Ops &d) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      mfma(o, q);
#pragma unroll
      for (int w = q * W / NM; w < (q + 1) * W / NM; ++w) odd_item(u, i, d, w >> 1, w & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // A clean step whose slice-0 operands are already in op0: slices 1.. of
  // u, and slice 0 of the following step un (unused after the last step:
  // its registers then hold a re-read step).
  auto run_step = [&](const Buf &u, const Buf &un) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kHW; ++i) {
      slice_odd_next(op0, u, i, op1);
      if (i + 1 < kHW)
        slice_even_next(op1, u, i + 1, op0, false);
      else
        slice_even_next(op1, un, 0, op0, true);
    }
  };
  // One slice on its own, pad elements masked in A (the steps after the
  // pipelined loop).
  auto unpack_masked = [&](const Buf &u, int j, Ops &o, int s) __attribute__((always_inline)) {
    const int64_t e = (int64_t)(s * kSW + kHW * h + (j >> 1)) * 64 + 32 * (j & 1);
    const uint32_t v = valid_bits(e, K);
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      const v4i c = fp4_chunk(u[p][j], c8, c2);
      o.s[p] = p < RB ? mask4(c, v) : c;
    }
  };

  // Two step register sets in ping-pong: the loads of step s+1 are issued
  // at the start of step s (a scheduling barrier keeps them there), and its
  // first slice is unpacked during step s's last one.  The loop runs whole
  // pairs of clean steps; the load past the last pair re-reads its second
  // step (in bounds, unused).  What is left -- an odd clean step and the
  // partial last step (K not a multiple of 64 * SW) -- runs after the loop
  // one slice at a time with the pad elements masked in A (a clean step's
  // mask keeps every element).
  Buf u0, u1;
  const int npair = nclean >> 1;
  if (npair > 0) {
    load_step(0, u0);
#pragma unroll
    for (int w = 0; w < W; ++w) even_item(u0, 0, op0, false, w >> 1, w & 1);
    for (int s = 0; s < 2 * npair; s += 2) {
      load_step(s + 1, u1);
      __builtin_amdgcn_sched_barrier(0);
      run_step(u0, u1);
      load_step(s + 2 < 2 * npair ? s + 2 : s + 1, u0);
      __builtin_amdgcn_sched_barrier(0);
      run_step(u1, u0);
    }
  }
  for (int s = 2 * npair; s < nsteps; ++s) {
    load_step(s, u0);  // words past K: garbage (masked) or 0 (past the rows)
#pragma unroll
    for (int j = 0; j < 2 * kHW; ++j) {
      unpack_masked(u0, j, op0, s);
#pragma unroll
      for (int q = 0; q < NM; ++q) mfma(op0, q);
    }
  }
}

template <int EPI, int WR, int WC, int RB, int CB, int SW, int MINB>
__global__ void __launch_bounds__(256, MINB)
    gemm_mfma_kernel(const uint64_t *__restrict__ xp, const uint64_t *__restrict__ wp,
                     const EpiParams ep, void *__restrict__ yv, int M, int N, int K, int kw,
                     int tiles_m, int tiles_n) {
  static_assert(WR * WC == 4, "4 waves per block");
  static_assert(!is_repack(EPI) || CB % 2 == 0, "repack pairs 32-column tiles");
  static_assert(SW == 4 || SW == 8, "two or four words per lane per step");
  constexpr int BM = WR * RB * 32, BN = WC * CB * 32;
  constexpr int kHW = SW / 2;  // words per step and lane
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // XCD-aware tile order (column-tile major: consecutive tiles share W).
  // Grids that are not a multiple of 8 keep the plain order past the last
  // whole group of 8.
  const int T = tiles_m * tiles_n;
  const int per = T >> 3;
  const int b = blockIdx.x;
  const int tile = b < (per << 3) ? (b & 7) * per + (b >> 3) : b;
  const int tn = tile / tiles_m, tm = tile - tn * tiles_m;
  const int mb = tm * BM, nb = tn * BN;  // block origin
  const int m0 = mb + (wave / WC) * (RB * 32);
  const int n0 = nb + (wave % WC) * (CB * 32);
  const int h = lane >> 5;    // which half of a step's words
  const int li = lane & 31;   // row / column within a 32 x 32 tile

  // Buffer resources over the block's rows of X and W: offsets are relative
  // to the block origin and the extent is exactly the rows that exist, so
  // every load past them returns 0.
  const int rows_a = (M - mb) < BM ? (M - mb) : BM;
  const int rows_b = (N - nb) < BN ? (N - nb) : BN;
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint64_t *>(xp + (int64_t)mb * kw), (short)0, rows_a * kw * 8, 0x00020000);
  const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint64_t *>(wp + (int64_t)nb * kw), (short)0, rows_b * kw * 8, 0x00020000);
  uint32_t aoff[RB], boff[CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    int r = m0 - mb + rb * 32 + li;
    r = r < rows_a ? r : rows_a - 1;  // rows past M compute garbage that is never stored
    aoff[rb] = (uint32_t)(r * kw * 8 + h * (kHW * 8));
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    int c = n0 - nb + cb * 32 + li;
    c = c < rows_b ? c : rows_b - 1;
    boff[cb] = (uint32_t)(c * kw * 8 + h * (kHW * 8));
  }

  // Per-column epilogue operands, fetched before the K loop.
  float a_pre[CB];
  uint64_t f_pre[CB / 2 > 0 ? CB / 2 : 1];
  {
    int nc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) nc[cb] = n0 + cb * 32;
    epilogue_operands<EPI, CB>(ep, nc, li, N, K, a_pre, f_pre);
  }
  v16f acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  // in VGPRs, opaque to the compiler, so that every mask is one
  // v_and_or_b32 (gfx9 VOP3 encodings take no literal)
  const uint32_t c8 = settled(0x88888888u), c2 = settled(0x22222222u);
  k_loop<RB, CB, SW>(acc, ares, bres, aoff, boff, K, kw, h, c8, c2);
  // Every load has been waited for before the stores (the compiler would
  // otherwise wait before each store).
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);

  // Epilogue.  acc[rb][cb][v] is the exact integer dot of row
  // m0 + rb*32 + 8(v/4) + 4h + v%4 and column n0 + cb*32 + li.
  int mr[RB], nc[CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) mr[rb] = m0 + rb * 32;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) nc[cb] = n0 + cb * 32;
  store_tiles<EPI, RB, CB>(acc, a_pre, f_pre, mr, nc, h, li, yv, M, N);
}


template <int EPI, int WR, int WC, int RB, int CB, int SW, int MINB>
hipError_t launch_cfg(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y, int M,
                      int N, int K, hipStream_t s) {
  constexpr int BM = WR * RB * 32, BN = WC * CB * 32;
  const int kw = (K + 63) / 64;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  hipLaunchKernelGGL((gemm_mfma_kernel<EPI, WR, WC, RB, CB, SW, MINB>), dim3((unsigned)tiles),
                     dim3(256), 0,
                     s, xp, wp, ep, y, M, N, K, kw, tiles_m, tiles_n);
  return hipGetLastError();
}

// Compute units of the current device (cached per device; 256 if the query
// fails, which only affects the choice of tile shape).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int EPI>
hipError_t launch_epi(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y, int M,
                      int N, int K, hipStream_t s) {
  // Narrow outputs stack the four waves along M so that no wave idles.
  if (N <= 64) return launch_cfg<EPI, 4, 1, 1, 2, 8, 2>(xp, wp, ep, y, M, N, K, s);  // 128 x 64
  // Large products: 256 x 256 block tiles of 4 x 4 wave tiles, while they
  // still give every CU at least one block and K is long enough for the K
  // loop (not the epilogue) to dominate a tile.  One block runs per CU, so
  // the tiles run in rounds of one per CU; when 320 x 192 block tiles (5 x 3
  // wave tiles: 15 instead of 16 MFMA tiles a wave, 2.93 instead of 2.75
  // unpack VALU per MFMA) need no more rounds, their shorter rounds win
  // (4096 x 11008: 754 tiles in 3 rounds against 688 in 3).  Repacked
  // outputs pair 32-column tiles and keep 4 x 4.
  const int64_t big = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  if (big >= 256 && K >= 2048) {
    if constexpr (!is_repack(EPI)) {
      const int64_t cus = cu_count();
      const int64_t t53 = (int64_t)((M + 319) / 320) * ((N + 191) / 192);
      const int64_t r44 = (big + cus - 1) / cus, r53 = (t53 + cus - 1) / cus;
      if (r53 * 31 < r44 * 32)  // rounds x tile work (15.5 against 16, the VALU counted in)
        return launch_cfg<EPI, 2, 2, 5, 3, 4, 1>(xp, wp, ep, y, M, N, K, s);
    }
    return launch_cfg<EPI, 2, 2, 4, 4, 4, 1>(xp, wp, ep, y, M, N, K, s);
  }
  return launch_cfg<EPI, 4, 1, 2, 2, 8, 2>(xp, wp, ep, y, M, N, K, s);  // 256 x 64
}

}  // namespace

hipError_t launch_gemm_mfma(const uint64_t *xp, const uint64_t *wp, const EpiParams &ep, void *y,
                            int64_t M, int64_t N, int64_t K, int epilogue, hipStream_t s) {
  switch (epilogue) {
    case BNN_EPI_I32:
      return launch_epi<BNN_EPI_I32>(xp, wp, ep, y, (int)M, (int)N, (int)K, s);
    case BNN_EPI_SCALED:
      return launch_epi<BNN_EPI_SCALED>(xp, wp, ep, y, (int)M, (int)N, (int)K, s);
    case kEpiRepackThr:
      return launch_epi<kEpiRepackThr>(xp, wp, ep, y, (int)M, (int)N, (int)K, s);
    default:
      return launch_epi<BNN_EPI_REPACK>(xp, wp, ep, y, (int)M, (int)N, (int)K, s);
  }
}

}  // namespace bnn
