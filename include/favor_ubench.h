/*
 * libfavor_ubench -- instruction-rate probes for the measurement of libfavor's
 * kernels.  Not part of the attention library: bench.py loads it to measure
 * the vector-unit rates that bound the feature-map kernels (every (token,
 * feature) pair of FAVOR+ needs one exponential, Performer notes, FAVOR+), so
 * that each kernel's time can be set against an exp/VALU floor beside its HBM
 * roofline.
 *
 * Each probe launches `blocks` workgroups of `threads` threads (threads a
 * multiple of 64, at most 1024); every thread runs `iters` iterations of 8
 * independent dependency chains and writes one float to out[global thread
 * index] (out holds blocks * threads floats, device memory, caller-owned), so
 * the work cannot be optimised away.  Per thread and iteration:
 *   favor_ubench_exp2 : 8 v_exp_f32 (x <- 2^-x on each chain; values stay in
 *                       [1/2, 1])
 *   favor_ubench_fma  : 8 v_fma_f32
 *   favor_ubench_mix  : 8 v_exp_f32 and 32 v_fma_f32, interleaved (shows
 *                       whether exponentials issue beside FMAs)
 * Returns 0, or 1 for invalid arguments (nothing launched), or 2 if the launch
 * failed.  Asynchronous on `stream`; time it with events on that stream.
 */
#ifndef FAVOR_UBENCH_H_
#define FAVOR_UBENCH_H_

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int favor_ubench_exp2(float* out, int blocks, int threads, int iters, hipStream_t stream);
int favor_ubench_fma(float* out, int blocks, int threads, int iters, hipStream_t stream);
int favor_ubench_mix(float* out, int blocks, int threads, int iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FAVOR_UBENCH_H_ */
