// api.hip -- the C-ABI of libbnn.so: host-side validation, kernel choice and
// status codes.  Every check runs before anything is enqueued, so an invalid
// call writes nothing and launches nothing.  No allocation, no
// synchronization, no state.
#include "../../include/bnn.h"
#include "bnn_internal.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;  // M, N, K, rows and ld limits
constexpr int64_t kGemvMaxM = 8;               // AUTO picks the GEMV kernel up to here

bool misaligned(const void *p, uintptr_t a) { return ((uintptr_t)p) % a != 0; }

bnn_status launch_status(hipError_t e) { return e == hipSuccess ? BNN_OK : BNN_E_LAUNCH; }

// Shared checks of the packed products; `epilogue` may be the internal
// threshold repack, whose operands `ep.thr` / `ep.flip` are checked here too.
bnn_status check_gemm(const uint64_t *xp, const uint64_t *wp, const bnn::EpiParams &ep,
                      const void *y, int64_t M, int64_t N, int64_t K, int epilogue, int algo) {
  if (epilogue < BNN_EPI_I32 || epilogue > bnn::kEpiRepackThr) return BNN_E_ARG;
  if (algo < BNN_ALGO_AUTO || algo > BNN_ALGO_MFMA) return BNN_E_ARG;
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return BNN_E_SHAPE;
  if (algo == BNN_ALGO_MFMA && K > bnn::kMfmaMaxK) return BNN_E_SHAPE;
  const int64_t kw = bnn_words(K);
  if ((M * kw > 0 && !xp) || (N * kw > 0 && !wp) || (M * N > 0 && !y)) return BNN_E_NULL;
  if (epilogue == BNN_EPI_SCALED && M * N > 0 && !ep.alpha) return BNN_E_NULL;
  if (epilogue == bnn::kEpiRepackThr && M * N > 0 && !ep.thr) return BNN_E_NULL;
  if (misaligned(xp, 8) || misaligned(wp, 8)) return BNN_E_ALIGN;
  if (misaligned(y, bnn::is_repack(epilogue) ? 8 : 4)) return BNN_E_ALIGN;
  if (epilogue == BNN_EPI_SCALED && misaligned(ep.alpha, 4)) return BNN_E_ALIGN;
  if (epilogue == bnn::kEpiRepackThr && (misaligned(ep.thr, 4) || misaligned(ep.flip, 8)))
    return BNN_E_ALIGN;
  return BNN_OK;
}

// Kernel choice and launch of a validated product.
bnn_status run_gemm(const uint64_t *xp, const uint64_t *wp, const bnn::EpiParams &ep, void *y,
                    int64_t M, int64_t N, int64_t K, int epilogue, int algo, hipStream_t s) {
  if (M == 0 || N == 0) return BNN_OK;
  if (algo == BNN_ALGO_AUTO) {
    if (K == 0)
      algo = BNN_ALGO_TILED;  // no K loop: the smallest kernel writes the constant result
    else if (M <= kGemvMaxM)
      algo = BNN_ALGO_GEMV;  // weight-streaming: HBM-bound
    else if (K <= bnn::kMfmaMaxK)
      algo = BNN_ALGO_MFMA;  // matrix cores: ~8x the VALU popcount rate
    else
      algo = BNN_ALGO_TILED;
  }
  if (algo == BNN_ALGO_GEMV)
    return launch_status(bnn::launch_gemv(xp, wp, ep, y, M, N, K, epilogue, s));
  if (algo == BNN_ALGO_MFMA)
    return launch_status(bnn::launch_gemm_mfma(xp, wp, ep, y, M, N, K, epilogue, s));
  return launch_status(bnn::launch_gemm_tiled(xp, wp, ep, y, M, N, K, epilogue, s));
}

}  // namespace

extern "C" {

int64_t bnn_words(int64_t k) { return k <= 0 ? 0 : (k + 63) / 64; }

const char *bnn_status_str(int status) {
  switch (status) {
    case BNN_OK: return "ok";
    case BNN_E_NULL: return "null pointer for a non-empty buffer";
    case BNN_E_SHAPE: return "invalid shape (negative, too large, or ld < k)";
    case BNN_E_DTYPE: return "unknown element type";
    case BNN_E_ALIGN: return "pointer not aligned to its element size";
    case BNN_E_LAUNCH: return "kernel launch failed";
    case BNN_E_ARG: return "unknown epilogue or algorithm selector";
    default: return "unknown status";
  }
}

const char *bnn_version(void) { return "bnn-mi355x 0.1 (gfx950)"; }

bnn_status bnn_pack_signs(const void *src, int dtype, int64_t rows, int64_t k, int64_t ld_src,
                          uint64_t *dst, void *stream) {
  if (dtype != BNN_FP32 && dtype != BNN_BF16) return BNN_E_DTYPE;
  if (rows < 0 || k < 0 || ld_src < k || rows >= kMaxDim || ld_src >= kMaxDim) return BNN_E_SHAPE;
  if (rows * k > 0 && !src) return BNN_E_NULL;
  if (rows * bnn_words(k) > 0 && !dst) return BNN_E_NULL;
  if (misaligned(src, dtype == BNN_FP32 ? 4 : 2) || misaligned(dst, 8)) return BNN_E_ALIGN;
  if (rows == 0 || k == 0) return BNN_OK;
  return launch_status(
      bnn::launch_pack(src, dtype, rows, k, ld_src, dst, static_cast<hipStream_t>(stream)));
}

bnn_status bnn_gemm_ex(const uint64_t *xp, const uint64_t *wp, const float *alpha, void *y,
                       int64_t M, int64_t N, int64_t K, int epilogue, int algo, void *stream) {
  if (epilogue < BNN_EPI_I32 || epilogue > BNN_EPI_REPACK) return BNN_E_ARG;
  const bnn::EpiParams ep{alpha, nullptr, nullptr};
  const bnn_status st = check_gemm(xp, wp, ep, y, M, N, K, epilogue, algo);
  if (st != BNN_OK) return st;
  return run_gemm(xp, wp, ep, y, M, N, K, epilogue, algo, static_cast<hipStream_t>(stream));
}

bnn_status bnn_gemm_sign_repack_thr(const uint64_t *xp, const uint64_t *wp, const int32_t *thr,
                                    const uint64_t *flip, uint64_t *yp, int64_t M, int64_t N,
                                    int64_t K, int algo, void *stream) {
  const bnn::EpiParams ep{nullptr, thr, flip};
  const bnn_status st = check_gemm(xp, wp, ep, yp, M, N, K, bnn::kEpiRepackThr, algo);
  if (st != BNN_OK) return st;
  return run_gemm(xp, wp, ep, yp, M, N, K, bnn::kEpiRepackThr, algo,
                  static_cast<hipStream_t>(stream));
}

bnn_status bnn_gemv_act(const void *x, int dtype, int64_t ldx, const uint64_t *wp,
                        const float *alpha, void *y, int64_t M, int64_t N, int64_t K, int epilogue,
                        void *stream) {
  if (dtype != BNN_FP32 && dtype != BNN_BF16) return BNN_E_DTYPE;
  if (epilogue < BNN_EPI_I32 || epilogue > BNN_EPI_REPACK) return BNN_E_ARG;
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim || ldx < K ||
      ldx >= kMaxDim)
    return BNN_E_SHAPE;
  const int64_t kw = bnn_words(K);
  if ((M * K > 0 && !x) || (N * kw > 0 && !wp) || (M * N > 0 && !y)) return BNN_E_NULL;
  if (epilogue == BNN_EPI_SCALED && M * N > 0 && !alpha) return BNN_E_NULL;
  if (misaligned(x, dtype == BNN_FP32 ? 4 : 2) || misaligned(wp, 8)) return BNN_E_ALIGN;
  if (misaligned(y, epilogue == BNN_EPI_REPACK ? 8 : 4)) return BNN_E_ALIGN;
  if (epilogue == BNN_EPI_SCALED && misaligned(alpha, 4)) return BNN_E_ALIGN;
  if (M == 0 || N == 0) return BNN_OK;
  const bnn::EpiParams ep{alpha, nullptr, nullptr};
  return launch_status(bnn::launch_gemv_act(x, dtype, ldx, wp, ep, y, M, N, K, epilogue,
                                            static_cast<hipStream_t>(stream)));
}

bnn_status bnn_gemm_signw_bf16(const void *x, int64_t ldx, const uint64_t *wp, const float *alpha,
                               float *y, int64_t M, int64_t N, int64_t K, int algo, void *stream) {
  if (algo != BNN_ALGO_AUTO && algo != BNN_ALGO_GEMV && algo != BNN_ALGO_MFMA) return BNN_E_ARG;
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim || ldx < K ||
      ldx >= kMaxDim)
    return BNN_E_SHAPE;
  const int64_t kw = bnn_words(K);
  if ((M * K > 0 && !x) || (N * kw > 0 && !wp) || (M * N > 0 && !y)) return BNN_E_NULL;
  if (misaligned(x, 2) || misaligned(wp, 8) || misaligned(y, 4) || misaligned(alpha, 4))
    return BNN_E_ALIGN;
  if (M == 0 || N == 0) return BNN_OK;
  const bool gemv_ok = bnn::signw_gemv_fits(M, K);
  if (algo == BNN_ALGO_GEMV && !gemv_ok) return BNN_E_SHAPE;
  if (algo == BNN_ALGO_AUTO) algo = gemv_ok ? BNN_ALGO_GEMV : BNN_ALGO_MFMA;
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (algo == BNN_ALGO_GEMV)
    return launch_status(bnn::launch_signw_gemv(xb, ldx, wp, alpha, y, M, N, K, s));
  return launch_status(bnn::launch_signw_mfma(xb, ldx, wp, alpha, y, M, N, K, s));
}

bnn_status bnn_chain3(const void *x, int dtype, int64_t ldx, const uint64_t *w1,
                      const int32_t *thr1, const uint64_t *flip1, const uint64_t *w2,
                      const int32_t *thr2, const uint64_t *flip2, const uint64_t *w3,
                      const float *alpha3, float *y, int64_t M, int64_t K0, int64_t N1, int64_t N2,
                      int64_t N3, void *stream) {
  if (dtype != BNN_FP32 && dtype != BNN_BF16) return BNN_E_DTYPE;
  if (M < 0 || M >= kMaxDim || ldx < K0 || ldx >= kMaxDim ||
      !bnn::chain3_dims_ok(K0, N1, N2, N3))
    return BNN_E_SHAPE;
  if ((M > 0 && (!x || !y)) || !w1 || !w2 || !w3) return BNN_E_NULL;
  if (misaligned(x, dtype == BNN_FP32 ? 4 : 2) || misaligned(w1, 8) || misaligned(w2, 8) ||
      misaligned(w3, 8) || misaligned(y, 4) || misaligned(alpha3, 4) || misaligned(thr1, 4) ||
      misaligned(thr2, 4) || misaligned(flip1, 8) || misaligned(flip2, 8))
    return BNN_E_ALIGN;
  if (M == 0) return BNN_OK;
  const bnn::Chain3Repack rp{thr1, flip1, thr2, flip2};
  return launch_status(bnn::launch_chain3(x, dtype, ldx, w1, w2, w3, alpha3, y, M, K0, N1, N2, N3,
                                          rp, static_cast<hipStream_t>(stream)));
}

bnn_status bnn_gemm_u64(const uint64_t *xp, const uint64_t *wp, int32_t *y, int64_t M, int64_t N,
                        int64_t K, void *stream) {
  return bnn_gemm_ex(xp, wp, nullptr, y, M, N, K, BNN_EPI_I32, BNN_ALGO_AUTO, stream);
}

bnn_status bnn_gemm_u64_scaled(const uint64_t *xp, const uint64_t *wp, const float *alpha,
                               float *y, int64_t M, int64_t N, int64_t K, void *stream) {
  return bnn_gemm_ex(xp, wp, alpha, y, M, N, K, BNN_EPI_SCALED, BNN_ALGO_AUTO, stream);
}

bnn_status bnn_gemm_sign_repack(const uint64_t *xp, const uint64_t *wp, uint64_t *yp, int64_t M,
                                int64_t N, int64_t K, void *stream) {
  return bnn_gemm_ex(xp, wp, nullptr, yp, M, N, K, BNN_EPI_REPACK, BNN_ALGO_AUTO, stream);
}

}  // extern "C"
