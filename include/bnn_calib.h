/*
 * bnn_calib.h -- C-ABI of libbnn_calib.so: rate probes that calibrate the
 * roofline fractions the benchmark reports for libbnn.so.  Not part of the
 * product path (libbnn.so neither links nor calls it).
 *
 * What they measure:
 *   - the issue rate of the VALU XOR + popcount pair on this GPU, the two
 *     instructions of one 64-bit word step of the packed product
 *     ("Binary Math Effectiveness -- why / how / when", section 2.1
 *     "Arithmetic": one XOR + popcount per 64-bit word);
 *   - the rate of the FP4 matrix-core instruction the large-M product runs
 *     on (v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands), with fixed
 *     operands and with +-1 operands that change from one MFMA to the next;
 *   - the read rate of HBM with the 16-byte non-temporal loads the
 *     weight-streaming kernels use (same page, sections 2.2-2.3: a batch-1
 *     product is bound by the bytes it streams);
 *   - the shader clock during each probe, from the shader cycle counter
 *     against the fixed-rate wall clock counter.
 *
 * Conventions: every pointer is a DEVICE pointer owned by the caller; each
 * call enqueues one kernel on `stream` (a hipStream_t, NULL = default) and
 * returns without synchronizing.  Errors: a non-zero status of the
 * bnn_status codes in bnn.h (BNN_E_NULL for a NULL `out`, BNN_E_SHAPE for
 * a non-positive count, BNN_E_ALIGN for an `out` not 8-byte aligned,
 * BNN_E_LAUNCH when the launch is rejected); nothing is enqueued then.
 *
 * Output record, per block, 4 int64 values written by the first lane of
 * the block's first wave:
 *   out[4*b + 0]  shader cycle counter (s_memtime) at the start of the loop
 *   out[4*b + 1]  shader cycle counter at the end of the loop
 *   out[4*b + 2]  wall clock counter (s_memrealtime) at the start
 *   out[4*b + 3]  wall clock counter at the end
 * and out[4*blocks] receives a value folded from every lane's result (so
 * that no work can be optimised away).  `out` must hold 4*blocks + 1
 * int64 values.
 */
#ifndef BNN_CALIB_H_
#define BNN_CALIB_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* VALU probe: `blocks` blocks of 256 threads; every thread runs `iters`
 * iterations of 4 rounds of 8 independent (v_xor_b32, v_bcnt_u32_b32)
 * pairs, i.e. 64 * iters 32-bit lane operations per thread. */
int bnn_calib_valu(int64_t *out, int64_t blocks, int64_t iters, void *stream);

/* Matrix-core probe: `blocks` blocks of 256 threads (4 waves); every wave
 * runs `iters` iterations of 4 independent FP4 32x32x64 MFMAs with unit
 * scales, i.e. 4 * iters * 131072 flops per wave. */
int bnn_calib_mfma_fp4(int64_t *out, int64_t blocks, int64_t iters, void *stream);

/* The same matrix-core probe on the data the packed product feeds: four
 * operand pairs of pseudo-random +-1 FP4 nibbles, and each of the 4 MFMAs
 * of an iteration takes another pair than the one before it (the rate of
 * the instruction depends on the operand bits it switches). */
int bnn_calib_mfma_fp4_pm1(int64_t *out, int64_t blocks, int64_t iters, void *stream);

/* HBM probe: `blocks` blocks of 256 threads read `bytes` bytes (a positive
 * multiple of 16) of `src` (16-byte aligned) once, 16 bytes per load with
 * non-temporal loads; each block step reads a contiguous 32 KiB chunk and the
 * blocks stride over the chunks: the practical read rate of this GPU's HBM
 * when the buffer is larger than the caches. */
int bnn_calib_read(const void *src, int64_t bytes, int64_t *out, int64_t blocks, void *stream);

/* Frequency of the wall clock counter in Hz (0 if the runtime cannot tell). */
int64_t bnn_calib_wallclock_hz(void);

#ifdef __cplusplus
}
#endif

#endif /* BNN_CALIB_H_ */
