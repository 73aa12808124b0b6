/*
 * fp8probe.h -- measurement probe shipped beside libfp8blk (libfp8probe.so).
 * Not part of the hot path: the benchmark uses it to state an on-box ceiling
 * for the block-scaled FP8 matrix-core work of the GEMM kernels.
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

#ifdef __cplusplus
}
#endif

#endif
