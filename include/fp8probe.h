/*
 * fp8probe.h -- measurement probe shipped beside libfp8blk (libfp8probe.so).
 * Not part of the hot path: the benchmark uses it to state on-box ceilings
 * for the block-scaled FP8 matrix-core work of the GEMM kernels and for the
 * HBM streaming of the quantizers, and a test uses it to check the
 * amax / 448 quantizers' quotient exhaustively.
 */
#ifndef FP8PROBE_H
#define FP8PROBE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue `workgroups` workgroups of 4 waves (one per SIMD when workgroups
 * <= 256 on MI355X), each issuing `iters` x 16 block-scaled 32x32x64 FP8
 * MFMAs on pseudo-random finite codes (seeded by `seed`), with the GEMM
 * kernels' accumulator layout.  out: device buffer of workgroups * 256
 * floats (a checksum per thread, so the work is not optimised away).
 * Returns 0, -1 for bad arguments, -6 if the launch failed.
 */
int fp8probe_mfma(int workgroups, int iters, uint32_t seed, float *out, hipStream_t stream);

/* The FLOP count of one fp8probe_mfma call (2 per multiply-add). */
double fp8probe_mfma_flops(int workgroups, int iters);

/*
 * On-box HBM ceiling: a streaming kernel over `bytes` (a multiple of 16;
 * src and dst 16-byte aligned) on `workgroups` workgroups of 256 threads,
 * each lane moving 8 16-byte pieces per step with non-temporal loads and
 * stores.  mode 0: copy src to dst (bytes read = bytes written, the
 * quantizers' ratio); mode 1: read src only, dst receiving one word per
 * thread (workgroups * 256 uint32) so that the loads are kept.
 * Returns 0, -1 for bad arguments, -6 if the launch failed.
 */
int fp8probe_stream(int mode, const void *src, void *dst, size_t bytes, int workgroups, hipStream_t stream);

/*
 * Check, on the device, the quantizers' quotient under FP8BLK_SCALE_FP32
 * against a plain IEEE division, for every element a quantizer can see:
 * every non-negative finite bf16 group amax a (bits 0 .. 0x7F7F) with every
 * bf16 x, |x| <= a, of either sign.  Both must give the same stored scale
 * fl32(a / 448) (1 for a = 0) and the same E4M3 code of x / s (clamped to
 * +-448).  counts: device buffer of FP8PROBE_QCHECK_BLOCKS uint32; entry
 * 128 a + j receives how many of the magnitudes 256 j .. 256 j + 255 differ.
 * Returns 0, -1 for a NULL buffer, -6 if the launch failed.
 */
#define FP8PROBE_QCHECK_BLOCKS (128 * 0x7F80)
int fp8probe_fp32_quotient_check(uint32_t *counts, hipStream_t stream);

/*
 * Check, on the device, the power-of-two quantizers' conversion (CDNA4's
 * v_cvt_scalef32_pk_fp8_bf16 given the stored scale s = 2^e) against the
 * exact product x * 2^-e rounded to E4M3 by v_cvt_pk_fp8_f32, for every
 * bf16 pattern x and every e in [-126, 126] with |x| * 2^-e <= 448 (each
 * result half of the instruction).  counts: device buffer of
 * FP8PROBE_CVTCHECK_BLOCKS uint32; entry 256 (e + 126) + j receives how many
 * of the bf16 patterns 256 j .. 256 j + 255 differ.  Returns 0, -1 for a
 * NULL buffer, -6 if the launch failed.
 */
#define FP8PROBE_CVTCHECK_BLOCKS (256 * 253)
int fp8probe_pow2_cvt_check(uint32_t *counts, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
