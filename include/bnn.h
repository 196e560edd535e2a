/*
 * bnn.h -- C-ABI of libbnn.so: packed binary (+1/-1) matrix products on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources cited by page title and section):
 *
 *   "Binary Math Effectiveness -- why / how / when", section 1 "The core
 *   identity":
 *     - encoding: a +1 is stored as bit 0 and a -1 as bit 1;
 *     - for x, w in {+1,-1}^n with d = popcount(x_bits XOR w_bits),
 *       <x, w> = n - 2d  (the library uses this XOR form);
 *     - edge cases: pad bits encode +1 and the identity uses the logical
 *       n, not 64 * words; n = 0 gives 0; a channel scale alpha = 0 gives a
 *       scaled output of 0; real inputs are projected to -1 when <= 0 and
 *       to +1 when > 0 before the identity is applied.
 *   Same page, section 2.1 "Arithmetic": a length-K row takes ceil(K/64)
 *   64-bit words, one XOR + popcount per word.
 *   Same page, sections 2.2-2.3: a batch-1 product is bound by the bytes of
 *   the weights it streams, 1/32 of fp32 when packed.
 *   "Architecture Decision Record" (Binary-Neural-Networks lab), Decision:
 *   matmuls are inferred with a packed XNOR/XOR + popcount kernel
 *   (binary_gemm_u64); this library is that operation for gfx950.
 *   "Encoder / decoder" (bnn/seq API), BinaryAutoEncoder: binary layers run
 *   back to back, which bnn_gemm_sign_repack serves by emitting the packed
 *   input of the next binary layer.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  X is M x K (activations, one row per token), W is N x K (one row
 * per output channel, nn.Linear orientation), Y = X * W^T is M x N.  All
 * matrices are dense row-major.  A packed matrix with R rows and K logical
 * columns is R x bnn_words(K) uint64 words, contiguous; logical element k
 * of a row is bit (k % 64) of word (k / 64), least significant bit first,
 * words little-endian in memory.
 *
 * Memory.  Every pointer is a DEVICE pointer owned by the caller.  The
 * library allocates nothing, frees nothing, keeps no state between calls
 * and never synchronizes: each call enqueues its kernels on `stream` (a
 * hipStream_t; NULL means the default stream) and returns.  Inputs and
 * outputs must not overlap.
 *
 * Pad bits.  Outputs that are packed (bnn_pack_signs, bnn_gemm_sign_repack)
 * have every pad bit 0 (+1).  Packed INPUTS may hold anything in their pad
 * bits: the kernels mask the last word, so only the K logical bits count.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued;
 * on error nothing is written or launched and a non-zero bnn_status is
 * returned.  A pointer may be NULL only when the buffer it names has no
 * elements.  M = 0 or N = 0 returns BNN_OK without a launch.  K = 0 is valid
 * and launches (dots are 0).  Dimensions (M, N, K, rows, leading
 * dimensions) must be >= 0 and < 2^30, else BNN_E_SHAPE.  A launch
 * failure reported by the HIP runtime right after the launch returns
 * BNN_E_LAUNCH; faults during execution surface at the caller's next
 * synchronization, as for any HIP kernel.
 *
 * Thread safety.  Calls are re-entrant and may be issued from several host
 * threads and on several streams at once.
 */
#ifndef BNN_H_
#define BNN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bnn_status {
  BNN_OK = 0,
  BNN_E_NULL = 1,   /* NULL pointer for a non-empty buffer */
  BNN_E_SHAPE = 2,  /* negative or too large dimension, ld < k, ... */
  BNN_E_DTYPE = 3,  /* unknown element type */
  BNN_E_ALIGN = 4,  /* pointer not aligned to its element size */
  BNN_E_LAUNCH = 5, /* the HIP runtime rejected a kernel launch */
  BNN_E_ARG = 6     /* unknown epilogue or algorithm selector */
} bnn_status;

typedef enum bnn_dtype {
  BNN_FP32 = 0, /* IEEE binary32 */
  BNN_BF16 = 1  /* bfloat16, the upper 16 bits of a binary32 */
} bnn_dtype;

/* Output stage of a product (see bnn_gemm_ex). */
typedef enum bnn_epilogue {
  BNN_EPI_I32 = 0,    /* int32 y = K - 2d */
  BNN_EPI_SCALED = 1, /* fp32 y = (float)(K - 2d) * alpha[n] */
  BNN_EPI_REPACK = 2  /* packed sign of (K - 2d) along N */
} bnn_epilogue;

/* Kernel family (see bnn_gemm_ex).  AUTO picks by shape. */
typedef enum bnn_algo {
  BNN_ALGO_AUTO = 0,  /* GEMV for M <= 8; MFMA for larger M while K <= 2^24;
                         TILED beyond */
  BNN_ALGO_GEMV = 1,  /* weight-streaming kernel; any M, fastest at M <= 8 */
  BNN_ALGO_TILED = 2, /* LDS-tiled VALU XOR + popcount GEMM; any K */
  BNN_ALGO_MFMA = 3   /* matrix-core GEMM: +-1 as FP4 operands, exact fp32
                         accumulation; K <= 2^24 (else BNN_E_SHAPE) */
} bnn_algo;

/* ceil(k / 64): 64-bit words per packed row of k logical values; 0 for
 * k <= 0.  ("Binary Math Effectiveness", section 2.1.) */
int64_t bnn_words(int64_t k);

/* Static, NUL-terminated description of a status code. */
const char *bnn_status_str(int status);

/* Static version string of the library. */
const char *bnn_version(void);

/*
 * bnn_pack_signs -- sign-project and pack along K.
 * ("Binary Math Effectiveness", section 1: encoding table and the edge-case
 * rows "padding" and "non-+-1 inputs".)
 *
 *   src     rows x ld_src elements of type `dtype` (BNN_FP32 or BNN_BF16),
 *           row-major; only the first k elements of each row are read.
 *   rows    number of rows (>= 0).
 *   k       logical row length (>= 0).
 *   ld_src  row stride of src in ELEMENTS (>= k).
 *   dst     rows x bnn_words(k) uint64 output, 8-byte aligned.
 *
 * Element v becomes bit 1 (-1) unless v > 0, in which case it becomes bit 0
 * (+1): +0, -0 and NaN give bit 1, positive subnormals give bit 0 (the test
 * is done on the bit pattern, so no flush-to-zero applies).  Pad bits of
 * each row's last word are written as 0.
 * Errors: BNN_E_NULL, BNN_E_SHAPE (negative sizes, ld_src < k),
 * BNN_E_DTYPE, BNN_E_ALIGN (src not aligned to its element, dst not 8-byte
 * aligned), BNN_E_LAUNCH.
 */
bnn_status bnn_pack_signs(const void *src, int dtype, int64_t rows, int64_t k, int64_t ld_src,
                          uint64_t *dst, void *stream);

/*
 * bnn_gemm_u64 -- y[m][n] = <x_m, w_n> = K - 2 * popcount(x_m XOR w_n) over
 * the K logical bits.  ("Binary Math Effectiveness", section 1, the core
 * identity and its edge cases; "Architecture Decision Record", Decision.)
 *
 *   xp  M x bnn_words(K) packed activations, 8-byte aligned.
 *   wp  N x bnn_words(K) packed weights, 8-byte aligned.
 *   y   M x N int32 output, row-major, 4-byte aligned.
 * K = 0 gives y = 0.  Errors: BNN_E_NULL, BNN_E_SHAPE, BNN_E_ALIGN,
 * BNN_E_LAUNCH.
 */
bnn_status bnn_gemm_u64(const uint64_t *xp, const uint64_t *wp, int32_t *y, int64_t M, int64_t N,
                        int64_t K, void *stream);

/*
 * bnn_gemm_u64_scaled -- y[m][n] = (float)(K - 2d) * alpha[n], one fp32
 * multiply rounded to nearest even (the integer converts exactly while
 * |K - 2d| <= 2^24).  ("Binary Math Effectiveness", section 1, edge case
 * "channel scale alpha"; alpha = 0 gives 0.)
 *
 *   alpha  N fp32 per-output-channel scales, 4-byte aligned.
 *   y      M x N fp32 output, row-major, 4-byte aligned.
 * Other arguments and errors as bnn_gemm_u64.
 */
bnn_status bnn_gemm_u64_scaled(const uint64_t *xp, const uint64_t *wp, const float *alpha,
                               float *y, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * bnn_gemm_sign_repack -- the packed input of the next binary layer:
 * bit n of output row m is 1 (-1) when K - 2d <= 0 and 0 (+1) otherwise,
 * packed along N exactly as bnn_pack_signs packs along K.  ("Binary Math
 * Effectiveness", section 1, the projection rule applied to a layer's
 * integer output; "Encoder / decoder", BinaryAutoEncoder, for chained
 * binary layers.)
 *
 *   yp  M x bnn_words(N) uint64 output, 8-byte aligned; pad bits are 0.
 * K = 0 gives dots of 0 and hence every logical bit 1.  Other arguments and
 * errors as bnn_gemm_u64.
 */
bnn_status bnn_gemm_sign_repack(const uint64_t *xp, const uint64_t *wp, uint64_t *yp, int64_t M,
                                int64_t N, int64_t K, void *stream);

/*
 * bnn_gemm_sign_repack_thr -- sign -> repack against a per-output-channel
 * integer threshold, with an optional per-channel flip: bit n of output row
 * m is 1 (-1) when (K - 2d) <= thr[n], inverted where bit n of `flip` is 1.
 * This is the form a BatchNorm placed after a binary layer takes when it is
 * folded into the projection that feeds the next binary layer
 * ("Architecture Decision Record", Decision: BN after the binary layers):
 * with z = g*(a*dot - mu)/s + b, a positive slope g*a/s projects to -1
 * exactly when dot <= floor(tau), tau = (mu - b*s/g)/a, and a negative slope
 * exactly when not (dot <= ceil(tau) - 1), which is the flipped form.
 * thr = 0 with no flip is bnn_gemm_sign_repack.
 *
 *   thr   N int32 thresholds, 4-byte aligned (any value; those >= K make
 *         every dot pass, those < -K none).
 *   flip  bnn_words(N) uint64 flip mask, bit n of word n/64 for channel n
 *         (the bnn_pack_signs layout of a length-N row), 8-byte aligned, or
 *         NULL for no flips.  Bits past N are ignored.
 *   yp    M x bnn_words(N) uint64 output, 8-byte aligned; pad bits are 0.
 *   algo  a BNN_ALGO_* value, as for bnn_gemm_ex (all bit-identical).
 * Errors as bnn_gemm_u64, plus BNN_E_NULL for a NULL thr with M*N > 0 and
 * BNN_E_ARG for an unknown algo.
 */
bnn_status bnn_gemm_sign_repack_thr(const uint64_t *xp, const uint64_t *wp, const int32_t *thr,
                                    const uint64_t *flip, uint64_t *yp, int64_t M, int64_t N,
                                    int64_t K, int algo, void *stream);

/*
 * bnn_gemm_signw_bf16 -- real-valued bf16 activations times packed sign
 * weights: y[m][n] = alpha[n] * sum_{k<K} x[m][k] * w_n[k], with w_n[k] = +1
 * for bit 0 and -1 for bit 1 of packed row n (the bnn_pack_signs layout).
 * This is the inference form of a layer whose weights alone are binarised
 * (binary_nn README, "Binary Regression" and "Triton Kernel Benchmark": the
 * eval-only packed-sign path of BinaryLinear); the weights keep their 1-bit
 * form ("Binary Math Effectiveness", section 2.2), the activations stay real.
 *
 * Arithmetic: every product x*(+-1) is exact; the K-term sum is accumulated
 * in fp32 in an order the kernel chooses (a tree of v_dot2 / MFMA partial
 * sums), then multiplied by alpha[n] once.  The result therefore differs
 * from the exact value by fp32 summation rounding only: at most
 * |alpha| * gamma * sum_k |x[m][k]| + 2^-23 |y|, gamma = K 2^-23 / (1 - K 2^-23),
 * and it is exact whenever every partial sum is representable in fp32 (for
 * example integer-valued activations with |sum| < 2^24).  Inputs must be
 * finite.  Elements past K and pad bits are never used.
 *
 *   x      M rows of bf16 values (raw 16-bit patterns), row stride ldx >= K
 *          elements, 2-byte aligned.
 *   wp     N x bnn_words(K) packed sign weights, 8-byte aligned.
 *   alpha  N fp32 per-output-channel scales, 4-byte aligned, or NULL for
 *          none (alpha = 1; the sum is stored as is).
 *   y      M x N fp32 output, row-major, 4-byte aligned.
 *   algo   BNN_ALGO_AUTO, BNN_ALGO_GEMV (small M: M <= 8 and the rows fit in
 *          64 KiB of LDS, else BNN_E_SHAPE) or BNN_ALGO_MFMA (any shape; bf16
 *          matrix cores).  The two kernels sum in different orders, so
 *          their results may differ by rounding.  BNN_ALGO_TILED -> BNN_E_ARG.
 * K = 0 gives y = 0 (times alpha).  Errors: BNN_E_SHAPE (negative or too
 * large sizes, ldx < K), BNN_E_NULL, BNN_E_ALIGN, BNN_E_ARG, BNN_E_LAUNCH.
 */
bnn_status bnn_gemm_signw_bf16(const void *x, int64_t ldx, const uint64_t *wp, const float *alpha,
                               float *y, int64_t M, int64_t N, int64_t K, int algo, void *stream);

/*
 * bnn_chain3 -- three chained binary layers in one launch: the M real-valued
 * input rows x (fp32 or bf16, K0 columns, row stride ldx) are sign-projected
 * and packed; layer 1 (w1: N1 x bnn_words(K0)) and layer 2 (w2: N2 x
 * bnn_words(N1)) end in sign -> repack; layer 3 (w3: N3 x bnn_words(N2))
 * ends in fp32, times alpha3[n] when alpha3 is non-NULL.  The result is bit
 * for bit that of bnn_pack_signs, bnn_gemm_sign_repack (twice; or
 * bnn_gemm_sign_repack_thr with the thresholds below) and
 * bnn_gemm_u64_scaled (or the int32 dot as fp32 when alpha3 is NULL); the
 * packed hidden activations stay on chip.  ("Encoder / decoder",
 * BinaryAutoEncoder, and the balanced_ternary_engine README 512 -> 256 ->
 * 128 -> 64 stack, for chained binary layers; "Binary Math Effectiveness",
 * section 1, for every step.)
 *
 *   x        M x ldx values of type dtype (BNN_FP32 / BNN_BF16), ldx >= K0,
 *            element-aligned.
 *   w1..w3   packed weights as above, 8-byte aligned.
 *   thr1, flip1 / thr2, flip2
 *            optional threshold repack of hidden layer 1 / 2, exactly as
 *            bnn_gemm_sign_repack_thr: int32 thresholds per output channel
 *            (N1 / N2 of them, 4-byte aligned) and packed flip masks
 *            (bnn_words(N1) / bnn_words(N2) words, 8-byte aligned); either
 *            may be NULL (threshold 0 / no flips), so all NULL is the plain
 *            sign -> repack.  A BatchNorm after each hidden binary layer
 *            folds into them ("Architecture Decision Record", Decision).
 *   alpha3   N3 fp32 scales, 4-byte aligned, or NULL.
 *   y        M x N3 fp32 output, row-major, 4-byte aligned.
 * Supported layer sizes: K0, N1, N2 in {128, 256, 384, 512}; N3 a multiple
 * of 32 in [32, 512]; otherwise BNN_E_SHAPE (use the separate calls).
 * M = 0 launches nothing.  Errors: BNN_E_DTYPE, BNN_E_SHAPE, BNN_E_NULL,
 * BNN_E_ALIGN, BNN_E_LAUNCH.
 */
bnn_status bnn_chain3(const void *x, int dtype, int64_t ldx, const uint64_t *w1,
                      const int32_t *thr1, const uint64_t *flip1, const uint64_t *w2,
                      const int32_t *thr2, const uint64_t *flip2, const uint64_t *w3,
                      const float *alpha3, float *y, int64_t M, int64_t K0, int64_t N1, int64_t N2,
                      int64_t N3, void *stream);

/*
 * bnn_gemm_ex -- the general form of the three products above, with an
 * explicit kernel family (see bnn_algo; the matrix-core family takes the
 * same exact integer sum of +-1 products on the MFMA units, which "Binary
 * Math Effectiveness", section 3, names as the faster dense unit).  `y` is int32*, float* or uint64* according to
 * `epilogue` (BNN_EPI_*); `alpha` is read only for BNN_EPI_SCALED.  `algo`
 * is a BNN_ALGO_* value; every family gives bit-identical results, so the
 * selector only changes speed.  Errors as above, plus BNN_E_ARG for an
 * unknown epilogue or algo.
 */
bnn_status bnn_gemm_ex(const uint64_t *xp, const uint64_t *wp, const float *alpha, void *y,
                       int64_t M, int64_t N, int64_t K, int epilogue, int algo, void *stream);

/*
 * bnn_gemv_act -- the weight-streaming product for small M with the
 * activation packing fused in: x holds M real-valued rows (fp32 or bf16,
 * row stride ldx elements, ldx >= K), which the kernel sign-projects and
 * packs exactly as bnn_pack_signs would before taking the product with the
 * packed weights wp.  The result equals bnn_pack_signs followed by
 * bnn_gemm_ex with the same epilogue, bit for bit.  ("Binary Math
 * Effectiveness", section 1, for the projection and the identity;
 * sections 2.2-2.3 for the batch-1 regime it serves: one launch per
 * decode step, weights streamed once.)
 *
 *   x         M x ldx values of type `dtype`, element-aligned.
 *   wp        N x bnn_words(K) packed weights, 8-byte aligned.
 *   alpha, y  as for bnn_gemm_ex with `epilogue`.
 * Intended for M <= 8; larger M is correct but streams W once per 8 rows
 * (pack once with bnn_pack_signs and use bnn_gemm_ex instead).  Errors as
 * bnn_gemm_ex, plus BNN_E_DTYPE, and BNN_E_SHAPE when ldx < K.
 */
bnn_status bnn_gemv_act(const void *x, int dtype, int64_t ldx, const uint64_t *wp,
                        const float *alpha, void *y, int64_t M, int64_t N, int64_t K, int epilogue,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BNN_H_ */
